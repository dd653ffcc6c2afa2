/*
 * ORACLE — test infrastructure, not part of the product.
 *
 * A plain, slow, obviously correct CPU implementation of what the W2A8 linear
 * layer computes.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load it.  It shares no code, header, table or constant
 * generator with the GPU library; neither side includes the other.
 *
 * Sources (cited by page title and section):
 *   [WIN]  "Windows 上跑通 BitNet b1.58：Flash Attention 与 CUDA sm_86 部署实录",
 *          §3.1 "BitLinear 层的三元权重逻辑".
 *   [CPU]  "微软BitNet：1-bit量化大模型CPU部署实践",
 *          §2.1 "1.58-bit量化原理", §2.2 "CPU优化设计", §6.3 "模型微调".
 *   [DEPLOY] "使用 BitNet 框架部署 1-bit LLM：三元权重量化、LUT 矩阵乘加速与
 *          GPU 运行时优化", section "GPU 运行时优化与低延迟推理管道".
 *   [TEST] "如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？",
 *          sections "运行 test.py 做 GEMV 基准测试", "如何判断结果",
 *          "限制与注意事项".
 *
 * Precision: integer work is exact (int64 accumulation).  Floating-point
 * steps use the precision the readings below fix (fp32 IEEE operations,
 * round-to-nearest-even, no contraction; sums of |W| in fp64).  Build with
 * -ffp-contract=off and without -ffast-math.
 *
 * Parity status of every function is stated in its comment; all are pinned
 * by the not-gpu tests (closed forms, invariants, brute force, worked
 * examples derived by hand from the definitions).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* O1. Integer product.
 *
 * [TEST] "运行 test.py 做 GEMV 基准测试" / "如何判断结果": the kernel's output
 * must equal the integer matrix product of the int8 activations and the
 * weights element by element.  [CPU] §2.1: with weights in {-1, 0, 1} each
 * product is an add, a skip or a subtract, so the result is the plain sum.
 * [TEST] "限制与注意事项": M is the number of tokens (M == 1 is decode).
 *
 *   y[m][n] = sum_{k<K} x[m][k] * w[n][k]
 *
 * x: int8 [M][K] row-major; w: int8 [N][K] row-major; y: int32 [M][N].
 * Returns 0, or -1 if a sum does not fit int32 (never for |x| <= 128,
 * |w| <= 1, K < 2^24).
 */
int oracle_gemm_i32(const int8_t *x, const int8_t *w, int64_t M, int64_t N,
                    int64_t K, int32_t *y)
{
    for (int64_t m = 0; m < M; ++m) {
        const int8_t *xr = x + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *wr = w + n * K;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)xr[k] * (int64_t)wr[k];
            if (acc > INT32_MAX || acc < INT32_MIN)
                return -1;
            y[m * N + n] = (int32_t)acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O2. Absmean ternarization of a full-precision weight matrix.
 *
 * [WIN] §3.1: the scale is the mean of the absolute values of the whole
 * weight matrix; each weight is divided by it and rounded to -1, 0 or 1.
 * [CPU] §6.3 gives the same with an explicit clamp:
 *   scale = mean(|W|);  Wq = clamp(round(W / scale), -1, 1).
 *
 * Readings (pages silent on these):
 *   - the mean is accumulated in fp64 in row-major order and rounded once to
 *     fp32 (the fp32 scale is what the epilogue multiplies back);
 *   - W / scale is an fp32 IEEE division; round is round-half-to-even (the
 *     page's torch.round rounds half to even);
 *   - an all-zero matrix gives scale 0 and Wq = 0 (no division happens).
 */
void oracle_ternarize_absmean(const float *W, int64_t N, int64_t K,
                              int8_t *wq, float *sw_out)
{
    const int64_t total = N * K;
    double s = 0.0;
    for (int64_t i = 0; i < total; ++i)
        s += fabs((double)W[i]);
    const float sw = total > 0 ? (float)(s / (double)total) : 0.0f;
    *sw_out = sw;
    for (int64_t i = 0; i < total; ++i) {
        if (sw == 0.0f) {
            wq[i] = 0;
            continue;
        }
        volatile float q = W[i] / sw;      /* fp32 division, stored as fp32 */
        float r = nearbyintf(q);           /* default mode: nearest, ties to even */
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        wq[i] = (int8_t)r;
    }
}

/* ------------------------------------------------------------------------ */
/* O3. Per-token absmax quantization of bf16 activations to int8.
 *
 * [TEST] (page intro): the kernels take 8-bit activations; no page gives the
 * quantizer.  Reading: per token (row m)
 *   a     = max_k |x[m][k]|             (bf16 -> fp32 is exact)
 *   inv   = 127 / a                     (fp32 division), capped at FLT_MAX
 *   q     = clamp(rne(x * inv), -127, 127)   (fp32 multiply, then round)
 *   sa[m] = a / 127                     (fp32 division, not 1/inv)
 * A row of zeros gives q = 0 and sa = 0.  The cap only matters for rows whose
 * maximum is below 127 / FLT_MAX (about 3.7e-37, subnormal-scale bf16): there
 * 127 / a overflows to infinity and 0 * inf would make the row's zeros NaN;
 * capped, zeros stay 0 and every code stays finite.  NaN / Inf inputs are
 * outside the contract.
 */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

void oracle_quant_act(const uint16_t *xb, int64_t M, int64_t K, int8_t *xq,
                      float *sa)
{
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = xb + m * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(bf16_to_f32(row[k]));
            if (v > a) a = v;
        }
        if (a == 0.0f) {
            for (int64_t k = 0; k < K; ++k) xq[m * K + k] = 0;
            sa[m] = 0.0f;
            continue;
        }
        volatile float inv = 127.0f / a;
        if (inv > FLT_MAX) inv = FLT_MAX;
        for (int64_t k = 0; k < K; ++k) {
            volatile float p = bf16_to_f32(row[k]) * inv;
            float r = nearbyintf(p);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            xq[m * K + k] = (int8_t)r;
        }
        volatile float s = a / 127.0f;
        sa[m] = s;
    }
}

/* ------------------------------------------------------------------------ */
/* O4. Scale epilogue.
 *
 * [WIN] §3.1: out = (round(W / scale) * x) * scale — the integer product is
 * computed first and the scale multiplied back afterwards.  With int8
 * activations x ~ xq * sa the layer output is acc * sa * sw.  Reading: two
 * fp32 multiplies, left to right, each rounded:
 *   y[m][n] = ((float)acc[m][n] * sa[m]) * sw
 */
void oracle_epilogue(const int32_t *acc, const float *sa, float sw, int64_t M,
                     int64_t N, float *y)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            volatile float t = (float)acc[m * N + n] * sa[m];
            volatile float r = t * sw;
            y[m * N + n] = r;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* a2. Ternary packing, element by element, from the layout definition.
 *
 * Code map: [CPU] §2.1 maps -1 -> 00, 0 -> 01, 1 -> 10, i.e. code = w + 1;
 * 11 is never produced.  Density: [CPU] §2.2 packs 8 ternary parameters into
 * 2 bytes (2 bits each).  [TEST] "编译 W2A8 CUDA 内核" says the reference
 * reorders the matrix in blocks and interleaves 16 2-bit values per 32-bit
 * word; its exact arrangement is not given, so the arrangement below is this
 * project's own ("T32x128", version 1):
 *
 *   Np = ceil(N/32)*32, Kp = ceil(K/128)*128, KT = Kp/128; Np*Kp/4 bytes.
 *   Element (n, k):
 *     s = n/32, r = n%32, rg = r/4, q = r%4          (row strip, group, word)
 *     t = k/128, c = k%128, kg = c/16, i = c%16       (k tile, group, index)
 *     j = i/4, b = i%4
 *     byte  = (s*KT + t)*1024 + (8*rg + kg)*16 + 4*q + b
 *     shift = 2*j   (bits shift..shift+1 of that byte hold the code)
 *   Positions with n >= N or k >= K hold code 01 (weight 0).
 *
 * oracle_pack returns 0, or -1 if a weight is outside {-1, 0, 1}.
 * oracle_unpack returns 0, or -1 if a code 11 is found inside the matrix.
 */
static int64_t ceil_to(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int64_t oracle_packed_bytes(int64_t N, int64_t K)
{
    return ceil_to(N, 32) * ceil_to(K, 128) / 4;
}

static void locate(int64_t n, int64_t k, int64_t KT, int64_t *byte, int *shift)
{
    int64_t s = n / 32, r = n % 32, rg = r / 4, q = r % 4;
    int64_t t = k / 128, c = k % 128, kg = c / 16, i = c % 16;
    int64_t j = i / 4, b = i % 4;
    *byte = (s * KT + t) * 1024 + (8 * rg + kg) * 16 + 4 * q + b;
    *shift = (int)(2 * j);
}

int oracle_pack(const int8_t *w, int64_t N, int64_t K, uint8_t *packed)
{
    const int64_t Np = ceil_to(N, 32), Kp = ceil_to(K, 128), KT = Kp / 128;
    /* every position starts as code 01 (weight 0): 0b01010101 per byte */
    memset(packed, 0x55, (size_t)(Np * Kp / 4));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int v = w[n * K + k];
            if (v < -1 || v > 1)
                return -1;
            int64_t byte;
            int shift;
            locate(n, k, KT, &byte, &shift);
            uint8_t code = (uint8_t)(v + 1);
            packed[byte] = (uint8_t)((packed[byte] & ~(3u << shift)) |
                                     ((unsigned)code << shift));
        }
    }
    return 0;
}

int oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *w)
{
    const int64_t KT = ceil_to(K, 128) / 128;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte;
            int shift;
            locate(n, k, KT, &byte, &shift);
            unsigned code = (packed[byte] >> shift) & 3u;
            if (code == 3u)
                return -1;
            w[n * K + k] = (int8_t)((int)code - 1);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O5. Per-token absmax int4 activation quantization (W2A4 variant).
 *
 * "使用 BitNet 框架部署 1-bit LLM：三元权重量化、LUT 矩阵乘加速与 GPU 运行时优化",
 * section "GPU 运行时优化与低延迟推理管道", names an "a4.8" extension with
 * lower-precision activations and gives no formula.
 * Reading: the O3 quantizer with 4-bit signed codes, 7 levels each side:
 *   a = max_k |x[m][k]|
 *   inv = 7 / a                         (fp32 division), capped at FLT_MAX
 *                                       as in O3 (a below 7 / FLT_MAX)
 *   q[m][k] = clamp(round_half_even(x[m][k] * inv), -7, 7)
 *   sa[m] = a / 7                       (fp32 division, not 1/inv)
 * A row of zeros gives q = 0 and sa = 0.  The product with ternary weights is
 * then O1 on these values, and the epilogue O4 with this sa.
 */
void oracle_quant_act_a4(const uint16_t *xb, int64_t M, int64_t K, int8_t *xq,
                         float *sa)
{
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = xb + m * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(bf16_to_f32(row[k]));
            if (v > a) a = v;
        }
        if (a == 0.0f) {
            for (int64_t k = 0; k < K; ++k) xq[m * K + k] = 0;
            sa[m] = 0.0f;
            continue;
        }
        volatile float inv = 7.0f / a;
        if (inv > FLT_MAX) inv = FLT_MAX;
        for (int64_t k = 0; k < K; ++k) {
            volatile float p = bf16_to_f32(row[k]) * inv;
            float r = nearbyintf(p);
            if (r > 7.0f) r = 7.0f;
            if (r < -7.0f) r = -7.0f;
            xq[m * K + k] = (int8_t)r;
        }
        volatile float s = a / 7.0f;
        sa[m] = s;
    }
}

/* ------------------------------------------------------------------------ */
/* a4 activation layout "A4I" (this project's own; the pages give none).
 *
 * Signed 4-bit values (two's complement nibbles, -8..7) of a row of K
 * activations, the row padded with zeros to a multiple of 32 values:
 * Kq = ceil(K/32)*32 values, Kq/2 bytes per row, rows back to back.
 * Element k of row m:
 *     c = k/16, i = k%16, h = i/4, j = i%4
 *     byte  = m*(Kq/2) + c*8 + 4*(h%2) + j
 *     shift = 4*(h/2)       (low nibble for h < 2, high nibble otherwise)
 * Why this order: in a T32x128 weight word (see the packing above) byte j
 * holds the codes of k = j, 4+j, 8+j, 12+j in bit pairs 0, 2, 4, 6.  The
 * masks 0x33333333 and (word>>2) & 0x33333333 put the codes of
 * {k = j, 8+j} and {k = 4+j, 12+j} into the nibbles of byte j, which are
 * exactly where this layout puts those activations in the chunk's first and
 * second 32-bit words.
 *
 * oracle_pack_act4 returns 0, or -1 if a value is outside -8..7.
 */
int64_t oracle_act4_bytes(int64_t M, int64_t K)
{
    return M * (ceil_to(K, 32) / 2);
}

static void locate4(int64_t m, int64_t k, int64_t K, int64_t *byte, int *shift)
{
    int64_t c = k / 16, i = k % 16, h = i / 4, j = i % 4;
    *byte = m * (ceil_to(K, 32) / 2) + c * 8 + 4 * (h % 2) + j;
    *shift = (int)(4 * (h / 2));
}

int oracle_pack_act4(const int8_t *q, int64_t M, int64_t K, uint8_t *out)
{
    memset(out, 0, (size_t)oracle_act4_bytes(M, K));
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            int v = q[m * K + k];
            if (v < -8 || v > 7)
                return -1;
            int64_t byte;
            int shift;
            locate4(m, k, K, &byte, &shift);
            out[byte] = (uint8_t)(out[byte] | (((unsigned)v & 15u) << shift));
        }
    }
    return 0;
}

void oracle_unpack_act4(const uint8_t *in, int64_t M, int64_t K, int8_t *q)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte;
            int shift;
            locate4(m, k, K, &byte, &shift);
            int v = (in[byte] >> shift) & 15;
            q[m * K + k] = (int8_t)(v >= 8 ? v - 16 : v);
        }
    }
}
