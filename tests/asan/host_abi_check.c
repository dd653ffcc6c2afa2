/* Host-side checks of libw2a8 for a build whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer (device code is compiled
 * as usual and never runs here).  Every buffer handed to the library is a
 * heap block of exactly the size the header documents, so a read or write
 * one byte past it is reported; the host arrays of the grouped entry points
 * hold exactly G entries for the same reason.  Device entry points are only
 * called with arguments the library rejects before it touches a device, or
 * (grouped, with valid host arrays) on a machine without a device, where
 * they end at the device query.
 *
 * Exit status 0 when every check holds; a sanitizer report aborts the run.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "w2a8.h"
#include "w2a8_tuning.h"

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* Pack, unpack and ternarize with exact-size buffers; ragged shapes leave
 * partial tiles at the bottom and right edges. */
static void check_weights(int64_t N, int64_t K) {
    const int64_t nb = w2a8_packed_bytes(N, K);
    CHECK(nb == ((N + 31) / 32) * 32 * ((K + 127) / 128) * 128 / 4);
    int8_t *w = xmalloc((size_t)(N * K));
    for (int64_t i = 0; i < N * K; ++i) w[i] = (int8_t)((int)(rnd() % 3) - 1);
    uint8_t *packed = xmalloc((size_t)nb);
    CHECK(pack_ternary(w, N, K, packed, nb) == W2A8_OK);
    CHECK(pack_ternary(w, N, K, packed, nb - 1) == W2A8_ERR_BUFSIZE);
    int8_t *back = xmalloc((size_t)(N * K));
    CHECK(unpack_ternary(packed, nb, N, K, back) == W2A8_OK);
    CHECK(memcmp(w, back, (size_t)(N * K)) == 0);
    CHECK(unpack_ternary(packed, nb - 1, N, K, back) == W2A8_ERR_BUFSIZE);
    w[N * K - 1] = 2;
    CHECK(pack_ternary(w, N, K, packed, nb) == W2A8_ERR_VALUE);

    float *W = xmalloc((size_t)(N * K) * sizeof(float));
    for (int64_t i = 0; i < N * K; ++i) W[i] = ((float)(rnd() % 2001) - 1000.0f) / 997.0f;
    float sw = -1.0f;
    CHECK(w2a8_ternarize_absmean(W, N, K, back, &sw) == W2A8_OK);
    CHECK(sw > 0.0f);
    for (int64_t i = 0; i < N * K; ++i) CHECK(back[i] >= -1 && back[i] <= 1);
    free(W);
    free(back);
    free(packed);
    free(w);
}

static void check_act_int4(int64_t M, int64_t K) {
    const int64_t nb = w2a4_act_bytes(M, K);
    CHECK(nb == M * ((K + 31) / 32) * 16);
    int8_t *q = xmalloc((size_t)(M * K));
    for (int64_t i = 0; i < M * K; ++i) q[i] = (int8_t)((int)(rnd() % 16) - 8);
    uint8_t *out = xmalloc((size_t)nb);
    CHECK(pack_act_int4(q, M, K, out, nb) == W2A8_OK);
    CHECK(pack_act_int4(q, M, K, out, nb - 1) == W2A8_ERR_BUFSIZE);
    q[0] = 8;
    CHECK(pack_act_int4(q, M, K, out, nb) == W2A8_ERR_VALUE);
    free(out);
    free(q);
}

/* Grouped entry points read exactly G entries of each host array. */
static void check_grouped(int G) {
    const void **wp = xmalloc(sizeof(void *) * (size_t)G);
    int64_t *N = xmalloc(sizeof(int64_t) * (size_t)G);
    float *sw = xmalloc(sizeof(float) * (size_t)G);
    int32_t **yi = xmalloc(sizeof(int32_t *) * (size_t)G);
    float **yf = xmalloc(sizeof(float *) * (size_t)G);
    for (int g = 0; g < G; ++g) {
        wp[g] = (const void *)(uintptr_t)(0x10000 + 0x1000 * g);
        N[g] = 32 * (g + 1) + g;
        sw[g] = 0.5f;
        yi[g] = (int32_t *)(uintptr_t)(0x80000 + 0x1000 * g);
        yf[g] = (float *)(uintptr_t)(0x100000 + 0x1000 * g);
    }
    const int8_t *x = (const int8_t *)(uintptr_t)0x200000;
    const float *sa = (const float *)(uintptr_t)0x210000;
    void *ws = (void *)(uintptr_t)0x220000;
    const int64_t K = 2560;
    /* valid host arrays: the call ends at the device query (no device here) */
    int st = w2a8_gemv_grouped(G, wp, N, K, x, sa, sw, yi, yf, ws, 1 << 20, NULL);
    CHECK(st == W2A8_ERR_NODEVICE || st == W2A8_ERR_ARCH);
    st = w2a8_linear_gemv_grouped(G, wp, N, K, (const uint16_t *)x, sw, yf, yi, ws, 1 << 20,
                                  NULL);
    CHECK(st == W2A8_ERR_NODEVICE || st == W2A8_ERR_ARCH);
    /* an invalid last entry is still read and rejected */
    N[G - 1] = 0;
    CHECK(w2a8_gemv_grouped(G, wp, N, K, x, sa, sw, yi, yf, ws, 1 << 20, NULL) ==
          W2A8_ERR_SHAPE);
    N[G - 1] = 64;
    yf[G - 1] = (float *)(uintptr_t)0x100004;
    CHECK(w2a8_gemv_grouped(G, wp, N, K, x, sa, sw, yi, yf, ws, 1 << 20, NULL) ==
          W2A8_ERR_ALIGN);
    st = w2a8_gemv_grouped(G, wp, N, K, x, sa, sw, yi, NULL, ws, 1 << 20, NULL);
    CHECK(st == W2A8_ERR_NODEVICE || st == W2A8_ERR_ARCH);
    free(yf);
    free(yi);
    free(sw);
    free(N);
    free(wp);
}

static void check_rejections(void) {
    const void *wp = (const void *)(uintptr_t)0x10000;
    const int8_t *x = (const int8_t *)(uintptr_t)0x20000;
    int32_t *y = (int32_t *)(uintptr_t)0x30000;
    float *yf = (float *)(uintptr_t)0x40000;
    const float *sa = (const float *)(uintptr_t)0x50000;
    void *ws = (void *)(uintptr_t)0x60000;
    CHECK(w2a8_gemv(NULL, x, 64, 2560, y, sa, 1.0f, yf, ws, 1 << 20, NULL) == W2A8_ERR_NULL);
    CHECK(w2a8_gemv(wp, x, 0, 2560, y, sa, 1.0f, yf, ws, 1 << 20, NULL) == W2A8_ERR_SHAPE);
    CHECK(w2a8_gemv(wp, x + 1, 64, 2560, y, sa, 1.0f, yf, ws, 1 << 20, NULL) == W2A8_ERR_ALIGN);
    CHECK(w2a8_gemv_noalloc(wp, x, 131073, 20480, y, sa, 1.0f, yf, NULL) == W2A8_ERR_SCRATCH);
    CHECK(w2a8_gemm(wp, x, 0, 64, 256, y, sa, 1.0f, yf, ws, 1 << 20, NULL) == W2A8_ERR_SHAPE);
    CHECK(w2a8_gemm(wp, x, 8, 64, 256, NULL, sa, 1.0f, NULL, ws, 1 << 20, NULL) ==
          W2A8_ERR_NULL);
    CHECK(quant_act_int8(NULL, 1, 256, (int8_t *)x, yf, NULL) == W2A8_ERR_NULL);
    CHECK(quant_act_int8((const uint16_t *)x, 1, 0, (int8_t *)x, yf, NULL) == W2A8_ERR_SHAPE);
    CHECK(w2a8_gemv_grouped(0, NULL, NULL, 256, x, sa, NULL, NULL, NULL, ws, 0, NULL) ==
          W2A8_ERR_SHAPE);
    CHECK(w2a8_gemv_grouped(W2A8_MAX_GROUPS + 1, NULL, NULL, 256, x, sa, NULL, NULL, NULL, ws,
                            0, NULL) == W2A8_ERR_SHAPE);
    for (int s = 0; s < 12; ++s) CHECK(w2a8_status_str(s) != NULL);
}

/* Plans and sizes over many shapes and device sizes. */
static void check_plans(void) {
    static const int64_t Ns[] = {1, 31, 32, 33, 2560, 6912, 27648, 55296, 131072};
    static const int64_t Ks[] = {1, 16, 127, 128, 129, 2560, 5120, 6016, 6144, 13824, 65536};
    static const int cus[] = {1, 32, 80, 256};
    for (size_t i = 0; i < sizeof Ns / sizeof *Ns; ++i)
        for (size_t j = 0; j < sizeof Ks / sizeof *Ks; ++j) {
            for (int64_t M = 1; M <= 20; ++M) CHECK(w2a8_workspace_bytes(M, Ns[i], Ks[j]) >= 0);
            for (size_t c = 0; c < sizeof cus / sizeof *cus; ++c) {
                int kernel = 0, wk = 0, sg = 0, depth = 0;
                CHECK(w2a8_gemv_plan(Ns[i], Ks[j], cus[c], &kernel, &wk, &sg, &depth) ==
                      W2A8_OK);
                CHECK(wk >= 1 && wk <= 16 && sg >= 1 && depth >= 1);
                /* kernel 3: sg counts its 8 row slices per strip, not k-ranges */
                if (kernel == 3) CHECK(wk == 1 && sg == 8 && Ks[j] % 16 == 0);
                else if (sg > 1) CHECK(w2a8_workspace_bytes(1, Ns[i], Ks[j]) > 0);
            }
        }
    int k = 0, wk = 0, sg = 0, d = 0;
    CHECK(w2a8_gemv_plan(0, 2560, 256, &k, &wk, &sg, &d) == W2A8_ERR_SHAPE);
    CHECK(w2a8_gemv_plan(2560, 2560, 256, NULL, &wk, &sg, &d) == W2A8_ERR_NULL);
}

/* Knob changes racing with plan reads (the knobs are read under a lock). */
static volatile int stop_flag = 0;
static void *flip_knobs(void *arg) {
    (void)arg;
    for (int i = 0; !__atomic_load_n(&stop_flag, __ATOMIC_RELAXED); ++i) {
        if (i & 1)
            w2a8_tune_gemv(1, 32, 2, 3, 1);
        else
            w2a8_tune_gemv(4, 6, 8, 256, 48);
        w2a8_tune_gemm(i % 5);
        w2a8_tune_gemm_ring((i & 2) ? 4 : 0, (i & 2) ? 3 : 0, (i & 2) ? 4 : 0);
    }
    return NULL;
}
static void *read_plans(void *arg) {
    (void)arg;
    for (int i = 0; i < 2000; ++i) {
        int k, wk, sg, d;
        if (w2a8_gemv_plan(5120, 27648, 256, &k, &wk, &sg, &d) != W2A8_OK) ++failures;
        if (w2a8_workspace_bytes(8, 5120, 27648) < 0) ++failures;
    }
    return NULL;
}
static void check_knob_threads(void) {
    pthread_t f, r[3];
    pthread_create(&f, NULL, flip_knobs, NULL);
    for (int i = 0; i < 3; ++i) pthread_create(&r[i], NULL, read_plans, NULL);
    for (int i = 0; i < 3; ++i) pthread_join(r[i], NULL);
    __atomic_store_n(&stop_flag, 1, __ATOMIC_RELAXED);
    pthread_join(f, NULL);
    CHECK(w2a8_tune_gemv(4, 6, 8, 256, 48) == W2A8_OK);
    CHECK(w2a8_tune_gemm(0) == W2A8_OK);
    CHECK(w2a8_tune_gemm_ring(0, 0, 0) == W2A8_OK);
}

int main(void) {
    static const int64_t shapes[][2] = {{1, 1},    {1, 128},  {31, 127}, {32, 128}, {33, 129},
                                        {64, 256}, {100, 1000}, {5, 8191}, {257, 384},
                                        {40, 2560}};
    for (size_t i = 0; i < sizeof shapes / sizeof *shapes; ++i)
        check_weights(shapes[i][0], shapes[i][1]);
    static const int64_t act[][2] = {{1, 1}, {1, 31}, {1, 32}, {3, 33}, {2, 2560}, {4, 1000}};
    for (size_t i = 0; i < sizeof act / sizeof *act; ++i) check_act_int4(act[i][0], act[i][1]);
    for (int G = 1; G <= W2A8_MAX_GROUPS; ++G) check_grouped(G);
    check_rejections();
    check_plans();
    check_knob_threads();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("host ABI checks passed\n");
    return 0;
}
