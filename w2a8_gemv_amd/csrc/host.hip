// Host side of libw2a8.so: argument validation, the offline steps
// (ternarization and packing) and the device entry points' dispatch.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "w2a8_tuning.h"

namespace w2a8 {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
bool g_dev_known[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];
int g_dev_status[kMaxDevices];

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool nk_ok(int64_t N, int64_t K) {
    return N >= 1 && K >= 1 && N <= kMaxN && K <= W2A8_MAX_K;
}

}  // namespace

int current_device(DeviceInfo *out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return W2A8_ERR_NODEVICE;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    if (!g_dev_known[dev]) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return W2A8_ERR_NODEVICE;
        DeviceInfo info;
        info.id = dev;
        info.cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
        info.xcds = 8;
        g_dev[dev] = info;
        g_dev_status[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? W2A8_OK : W2A8_ERR_ARCH;
        g_dev_known[dev] = true;
    }
    *out = g_dev[dev];
    return g_dev_status[dev];
}

int &gemm_kernel_mode() {
    static int mode = 0;
    return mode;
}

GemvPolicy &gemv_policy() {
    // Streaming kernel off by default (stream_min_tiles 0): on gfx950 the
    // workgroup kernel is as fast or faster on every measured shape.
    static GemvPolicy p = {4, 6, 8, 256, 48, 0, 4, 4};
    return p;
}

// Most workgroups a long strip is split into by default: more only for
// parallelism when there are few strips (each extra workgroup adds one atomic
// contribution per row).
constexpr int64_t kSplitWgs = 12;

// GEMV launch plan.
//  * SG workgroups share a 32-row strip (each one k-range of ktw tiles).  A
//    strip is split when it is long (KT >= split_min_tiles): into about one
//    workgroup per tiles_per_wave tiles, at most kSplitWgs, and into more
//    when there are too few strips to give wg_per_cu workgroups per CU.
//    Partials are combined with one device-scope atomic per row.
//    ktw <= krange_tiles always.
//  * A workgroup splits its range over WK <= 16 waves with runs of about
//    tiles_per_wave tiles (tiles_per_wave + 2 in a split strip, half of
//    tiles_per_wave in an unsplit strip when there are no more strips than
//    CUs; at most 32: each lane stages at most four 16-byte activation
//    chunks); their row sums are combined through LDS.  On those small grids
//    most CUs are idle and shorter runs finish sooner (measured on MI355X,
//    cold: 8 waves of 2-3 tiles against 4 waves of 5-7 tiles take 0.10 to
//    0.20 us less at 2560 x 2560, 3840 x 2560, 3200 x 3200 and 4800 x 3200;
//    at 55296 x 5120, 1728 strips, halving the runs costs 2.8 us).
//  * The load batch U (two in flight per wave) is the smallest of 2, 4, 8
//    (at most `unroll`) whose two batches cover the run.
void gemv_plan(int64_t NS, int64_t KT, int cus, int *wk, int *sg, int *run, int *unroll) {
    const GemvPolicy &p = gemv_policy();
    const int64_t tpw = std::max(1, p.tiles_per_wave);
    int64_t SG = ceil_div(KT, std::max(1, p.krange_tiles));
    if (KT >= p.split_min_tiles) {
        SG = std::max(SG, std::min(ceil_div(KT, tpw), kSplitWgs));
        const int64_t want = ceil_div(int64_t(cus) * std::max(1, p.wg_per_cu), NS);
        SG = std::max(SG, std::min(want, std::max<int64_t>(1, KT / tpw)));
    }
    SG = std::max<int64_t>(1, std::min(SG, KT));
    // Of SG and the two counts below it, the one whose k-ranges cover KT with
    // the fewest spare tiles (the larger count on a tie), so the workgroups of
    // a strip get equal ranges and fewer atomic contributions.  Measured on
    // MI355X, cold: 3200 x 10240 in 10 ranges of 8 tiles against 12 of 7
    // raised the 8-shape sweep from 1460 to 1477 GB/s (interleaved runs;
    // kernel-trace durations 4.92 against 5.18 us), though that shape
    // repeated on its own takes 0.07 us longer; 2560 x 27648 in 12 ranges of
    // 18 against 13 of 17: kernel-trace durations 6.52 against 6.92 us.
    if (SG > 2) {
        const int64_t lo = std::max<int64_t>(SG - 2, ceil_div(KT, std::max(1, p.krange_tiles)));
        int64_t best = SG, spare = ceil_div(KT, SG) * SG - KT;
        for (int64_t s = SG - 1; s >= lo && s >= 1; --s) {
            const int64_t sp = ceil_div(KT, s) * s - KT;
            if (sp < spare) {
                best = s;
                spare = sp;
            }
        }
        SG = best;
    }
    const int64_t ktw = ceil_div(KT, SG);
    // Runs of a split strip may be a little longer: its extra waves cost an
    // LDS combine on top of the atomic one.
    const int64_t run_tiles = SG > 1 ? tpw + 2 : NS <= cus ? std::max<int64_t>(1, tpw / 2) : tpw;
    int64_t WK = ceil_div(ktw, run_tiles);
    // An unsplit strip with more than two waves: a multiple of four, so the
    // workgroup spreads evenly over the compute unit's four SIMDs (5 or 7
    // waves measured slower than 4 or 8).
    if (SG == 1 && WK >= 3) WK = 4 * ((WK + 2) / 4);
    WK = std::min<int64_t>(WK, std::min<int64_t>(16, ktw));
    WK = std::max<int64_t>(WK, std::max<int64_t>(1, ceil_div(ktw, 32)));
    const int64_t R = ceil_div(ktw, WK);
    *wk = int(WK);
    *sg = int(SG);
    *run = int(R);
    const int u = R <= 4 ? 2 : R <= 8 ? 4 : 8;
    *unroll = std::min(u, p.unroll);
}

// Few activation rows: the GEMV plan with runs of at most 8 tiles (one
// activation chunk per lane per row) and at most 32/MR waves per workgroup
// (LDS <= 36 KiB for the MR row regions); more workgroups per strip when
// needed.
void gemv_rows_plan(int64_t NS, int64_t KT, int64_t M, int cus, int *wk, int *sg, int *run,
                    int *unroll) {
    int r = 0;
    gemv_plan(NS, KT, cus, wk, sg, &r, unroll);
    const int64_t MR = M <= 2 ? 2 : M <= 4 ? 4 : 8;
    const int64_t wkmax = 32 / MR;
    int64_t SG = *sg, WK = *wk;
    int64_t ktw = ceil_div(KT, SG);
    if (WK > wkmax || r > 8) {
        WK = std::min(wkmax, ceil_div(ktw, 8));
        if (ceil_div(ktw, WK) > 8) {
            SG = std::max(SG, ceil_div(KT, wkmax * 8));
            ktw = ceil_div(KT, SG);
            WK = std::min(wkmax, ceil_div(ktw, 8));
        }
        WK = std::max<int64_t>(1, std::min(WK, ktw));
    }
    const int64_t R = ceil_div(ktw, WK);
    *wk = int(WK);
    *sg = int(SG);
    *run = int(R);
    *unroll = R <= 4 ? 2 : 4;
}

// Large matrices (at least stream_min_tiles tiles, K staged whole in LDS)
// use the streaming kernel: a grid of CUs * stream_waves_per_cu long-lived
// waves, each streaming an equal contiguous share of the tiles.
void gemv_plan_full(int64_t NS, int64_t K, int cus, int *wk, int *sg, int *run, int *unroll,
                    int *g) {
    const GemvPolicy &p = gemv_policy();
    const int64_t KT = ceil_div(K, kTileK);
    const int64_t T = NS * KT;
    // (Tile indices are 32-bit in the streaming kernel: T < 2^30 is 1 TiB of weights.)
    if (p.stream_min_tiles > 0 && T >= p.stream_min_tiles && T < (int64_t(1) << 30) &&
        gemv_stream_fits(K)) {
        const int64_t G = std::min<int64_t>(T, int64_t(cus) * p.stream_waves_per_cu);
        *wk = *sg = *run = 0;
        *unroll = p.stream_unroll;
        *g = int(std::max<int64_t>(1, G));
        return;
    }
    *g = 0;
    gemv_plan(NS, KT, cus, wk, sg, run, unroll);
}

}  // namespace w2a8

using namespace w2a8;

extern "C" {

const char *w2a8_status_str(int status) {
    switch (status) {
    case W2A8_OK: return "ok";
    case W2A8_ERR_NULL: return "a required pointer is NULL";
    case W2A8_ERR_SHAPE: return "M, N or K out of range";
    case W2A8_ERR_ALIGN: return "a pointer is not aligned as required";
    case W2A8_ERR_VALUE: return "weight outside {-1,0,1} or invalid 2-bit code";
    case W2A8_ERR_BUFSIZE: return "packed or workspace buffer too small";
    case W2A8_ERR_NODEVICE: return "no HIP device available";
    case W2A8_ERR_ARCH: return "current device is not gfx950";
    case W2A8_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

int w2a8_layout_version(void) { return W2A8_LAYOUT_VERSION; }

int64_t w2a8_packed_bytes(int64_t N, int64_t K) {
    if (!nk_ok(N, K)) return -1;
    return round_up(N, kTileRows) * round_up(K, kTileK) / 4;
}

int64_t w2a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!nk_ok(N, K) || M < 1 || M > kMaxM) return -1;
    const int64_t Np = round_up(N, kTileRows);
    const int64_t NS = Np / kTileRows;
    int64_t bytes = 0;
    if (M == 1) {
        // GEMV: one 64-bit split-k combining word per padded row.
        bytes = 8 * Np;
    } else if (M <= kRowsMaxM) {
        // Few rows: a combining word per (row, padded output), or the general
        // kernel's split-K partials and counters, whichever is larger.
        bytes = std::max(8 * M * Np, 4 * M * Np + 4 * ceil_div(M, 16) * ceil_div(NS, 4));
    } else if (M * Np <= kGemmSplitMaxOut) {
        // GEMM split-K: int32 partial per output + one counter per
        // (m-block of >= 16 rows, n-block of 4 strips).
        bytes = 4 * M * Np + 4 * ceil_div(M, 16) * ceil_div(NS, 4);
    }
    return round_up(bytes, 256);
}

// ---------------------------------------------------------------------------
// a1: absmean ternarization (host)
// ---------------------------------------------------------------------------
int w2a8_ternarize_absmean(const float *W, int64_t N, int64_t K, int8_t *wq, float *sw) {
    if (!W || !wq || !sw) return W2A8_ERR_NULL;
    if (!nk_ok(N, K)) return W2A8_ERR_SHAPE;
    const int64_t total = N * K;
    // fp64 sum of |W| in row-major order, rounded once to fp32.
    double s = 0.0;
    for (int64_t i = 0; i < total; ++i) s += fabs(double(W[i]));
    const float scale = float(s / double(total));
    *sw = scale;
    if (scale == 0.0f) {
        memset(wq, 0, size_t(total));
        return W2A8_OK;
    }
    for (int64_t i = 0; i < total; ++i) {
        const float q = W[i] / scale;  // fp32 division
        float r = rintf(q);            // nearest, ties to even
        r = r > 1.0f ? 1.0f : (r < -1.0f ? -1.0f : r);
        wq[i] = int8_t(r);
    }
    return W2A8_OK;
}

// ---------------------------------------------------------------------------
// a2: packing (host).  One 32-bit word = 16 codes of one row.
// ---------------------------------------------------------------------------
int pack_ternary(const int8_t *w, int64_t N, int64_t K, void *packed, int64_t packed_bytes) {
    if (!w || !packed) return W2A8_ERR_NULL;
    if (!nk_ok(N, K)) return W2A8_ERR_SHAPE;
    const int64_t need = w2a8_packed_bytes(N, K);
    if (packed_bytes < need) return W2A8_ERR_BUFSIZE;
    const int64_t Np = round_up(N, kTileRows), KT = round_up(K, kTileK) / kTileK;
    uint32_t *out = static_cast<uint32_t *>(packed);
    for (int64_t n = 0; n < Np; ++n) {
        const int64_t s = n / kTileRows, r = n % kTileRows, rg = r / 4, q = r % 4;
        const int8_t *row = n < N ? w + n * K : nullptr;
        for (int64_t t = 0; t < KT; ++t) {
            uint32_t *tile = out + (s * KT + t) * kTileWords;
            for (int kg = 0; kg < 8; ++kg) {
                const int64_t k0 = t * kTileK + 16 * kg;
                uint32_t word = 0;
                for (int i = 0; i < 16; ++i) {
                    const int64_t k = k0 + i;
                    int v = 0;
                    if (row && k < K) {
                        v = row[k];
                        if (v < -1 || v > 1) return W2A8_ERR_VALUE;
                    }
                    const uint32_t code = uint32_t(v + 1);
                    word |= code << (8 * (i & 3) + 2 * (i >> 2));
                }
                tile[(8 * rg + kg) * 4 + q] = word;
            }
        }
    }
    return W2A8_OK;
}

int unpack_ternary(const void *packed, int64_t packed_bytes, int64_t N, int64_t K, int8_t *w) {
    if (!packed || !w) return W2A8_ERR_NULL;
    if (!nk_ok(N, K)) return W2A8_ERR_SHAPE;
    if (packed_bytes < w2a8_packed_bytes(N, K)) return W2A8_ERR_BUFSIZE;
    const int64_t KT = round_up(K, kTileK) / kTileK;
    const uint32_t *in = static_cast<const uint32_t *>(packed);
    for (int64_t n = 0; n < N; ++n) {
        const int64_t s = n / kTileRows, r = n % kTileRows, rg = r / 4, q = r % 4;
        for (int64_t t = 0; t < KT; ++t) {
            const uint32_t *tile = in + (s * KT + t) * kTileWords;
            for (int kg = 0; kg < 8; ++kg) {
                const uint32_t word = tile[(8 * rg + kg) * 4 + q];
                for (int i = 0; i < 16; ++i) {
                    const int64_t k = t * kTileK + 16 * kg + i;
                    if (k >= K) break;
                    const uint32_t code = (word >> (8 * (i & 3) + 2 * (i >> 2))) & 3u;
                    if (code == 3u) return W2A8_ERR_VALUE;
                    w[n * K + k] = int8_t(int(code) - 1);
                }
            }
        }
    }
    return W2A8_OK;
}

// ---------------------------------------------------------------------------
// a3: activation quantization (device)
// ---------------------------------------------------------------------------
int quant_act_int8(const uint16_t *x_bf16, int64_t M, int64_t K, int8_t *x_q, float *s_a,
                   void *stream) {
    if (!x_bf16 || !x_q || !s_a) return W2A8_ERR_NULL;
    if (M < 1 || M > kMaxM || K < 1 || K > W2A8_MAX_K) return W2A8_ERR_SHAPE;
    if (!aligned(x_bf16, 16) || !aligned(x_q, 16) || !aligned(s_a, 4)) return W2A8_ERR_ALIGN;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;
    hipError_t e = launch_quant(x_bf16, int(M), int(K), x_q, s_a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// a4..a7: GEMV (device)
// ---------------------------------------------------------------------------
int w2a8_gemv(const void *w_packed, const int8_t *x, int64_t N, int64_t K, int32_t *y_i32,
              const float *s_a, float s_w, float *y_f32, void *workspace, int64_t ws_bytes,
              void *stream) {
    if (!w_packed || !x || !workspace) return W2A8_ERR_NULL;
    if (!y_i32 && !y_f32) return W2A8_ERR_NULL;
    if (y_f32 && !s_a) return W2A8_ERR_NULL;
    if (!nk_ok(N, K)) return W2A8_ERR_SHAPE;
    if (!aligned(w_packed, 16) || !aligned(x, 16) || (y_i32 && !aligned(y_i32, 16)) ||
        (y_f32 && !aligned(y_f32, 16)) || (s_a && !aligned(s_a, 4)) || !aligned(workspace, 16))
        return W2A8_ERR_ALIGN;
    if (ws_bytes < w2a8_workspace_bytes(1, N, K)) return W2A8_ERR_BUFSIZE;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;

    const int64_t Np = round_up(N, kTileRows);
    GemvLaunch a;
    a.wp = static_cast<const uint32_t *>(w_packed);
    a.x = x;
    a.xb = nullptr;
    a.M = 1;
    a.y_i32 = y_i32;
    a.y_f32 = y_f32;
    a.sa = s_a;
    a.sw = s_w;
    a.ws_row = static_cast<uint64_t *>(workspace);
    a.N = int(N);
    a.K = int(K);
    a.KT = int(round_up(K, kTileK) / kTileK);
    a.NS = int(Np / kTileRows);
    gemv_plan_full(a.NS, K, dev.cus, &a.WK, &a.SG, &a.RUN, &a.unroll, &a.G);
    a.DXOK = int64_t(a.NS) * a.SG * a.WK <= 5 * int64_t(dev.cus);
    hipError_t e = a.G > 0 ? launch_gemv_stream(a, static_cast<hipStream_t>(stream))
                           : launch_gemv(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

// Fused linear layer for one token: quant_act_int8 + w2a8_gemv (fp32
// epilogue) in one launch.  Always the workgroup kernel.
int w2a8_linear_gemv(const void *w_packed, const uint16_t *x_bf16, int64_t N, int64_t K, float s_w,
                     float *y_f32, int32_t *y_i32, void *workspace, int64_t ws_bytes,
                     void *stream) {
    if (!w_packed || !x_bf16 || !y_f32 || !workspace) return W2A8_ERR_NULL;
    if (!nk_ok(N, K)) return W2A8_ERR_SHAPE;
    if (!aligned(w_packed, 16) || !aligned(x_bf16, 16) || !aligned(y_f32, 16) ||
        (y_i32 && !aligned(y_i32, 16)) || !aligned(workspace, 16))
        return W2A8_ERR_ALIGN;
    if (ws_bytes < w2a8_workspace_bytes(1, N, K)) return W2A8_ERR_BUFSIZE;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;

    const int64_t Np = round_up(N, kTileRows);
    GemvLaunch a;
    a.wp = static_cast<const uint32_t *>(w_packed);
    a.x = nullptr;
    a.xb = x_bf16;
    a.M = 1;
    a.y_i32 = y_i32;
    a.y_f32 = y_f32;
    a.sa = nullptr;
    a.sw = s_w;
    a.ws_row = static_cast<uint64_t *>(workspace);
    a.N = int(N);
    a.K = int(K);
    a.KT = int(round_up(K, kTileK) / kTileK);
    a.NS = int(Np / kTileRows);
    a.G = 0;
    gemv_plan(a.NS, a.KT, dev.cus, &a.WK, &a.SG, &a.RUN, &a.unroll);
    hipError_t e = launch_gemv_fused(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Grouped GEMV: several projections sharing x and K in one launch
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// Validates the projection arrays and fills the table; the launch's NS is
// the total strip count.  `need_f32` makes every y_f32 entry mandatory.
int grouped_setup(int G, const void *const *w_packed, const int64_t *N, int64_t K,
                  const float *s_w, int32_t *const *y_i32, float *const *y_f32, bool need_f32,
                  GemvGroups *t, int64_t *ns_total, int64_t *ws_need, bool *any_f32) {
    if (G < 1 || G > kMaxGroups) return W2A8_ERR_SHAPE;
    if (!w_packed || !N || !s_w) return W2A8_ERR_NULL;
    if (need_f32 && !y_f32) return W2A8_ERR_NULL;
    int64_t ns = 0, ws = 0;
    *any_f32 = false;
    for (int g = 0; g < G; ++g) {
        if (!nk_ok(N[g], K)) return W2A8_ERR_SHAPE;
        int32_t *yi = y_i32 ? y_i32[g] : nullptr;
        float *yf = y_f32 ? y_f32[g] : nullptr;
        if (!w_packed[g] || (!yi && !yf) || (need_f32 && !yf)) return W2A8_ERR_NULL;
        if (!aligned(w_packed[g], 16) || (yi && !aligned(yi, 16)) || (yf && !aligned(yf, 16)))
            return W2A8_ERR_ALIGN;
        *any_f32 = *any_f32 || yf != nullptr;
        const int64_t Np = round_up(N[g], kTileRows);
        t->begin[g] = int(ns);
        t->N[g] = int(N[g]);
        t->sw[g] = s_w[g];
        t->wp[g] = static_cast<const uint32_t *>(w_packed[g]);
        t->y_i32[g] = yi;
        t->y_f32[g] = yf;
        ns += Np / kTileRows;
        ws += w2a8_workspace_bytes(1, N[g], K);
        if (ns * kTileRows > kMaxN) return W2A8_ERR_SHAPE;
    }
    for (int g = G; g < kMaxGroups; ++g) {
        t->begin[g] = INT32_MAX;
        t->N[g] = 0;
        t->sw[g] = 0.0f;
        t->wp[g] = nullptr;
        t->y_i32[g] = nullptr;
        t->y_f32[g] = nullptr;
    }
    *ns_total = ns;
    *ws_need = ws;
    return W2A8_OK;
}

int grouped_launch(const GemvGroups &t, int64_t ns, int64_t K, const int8_t *x,
                   const uint16_t *xb, const float *s_a, void *workspace, void *stream) {
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;
    GemvLaunch a;
    a.wp = nullptr;
    a.x = x;
    a.xb = xb;
    a.M = 1;
    a.y_i32 = nullptr;
    a.y_f32 = nullptr;
    a.sa = s_a;
    a.sw = 0.0f;
    a.ws_row = static_cast<uint64_t *>(workspace);
    a.N = int(ns * kTileRows);
    a.K = int(K);
    a.KT = int(round_up(K, kTileK) / kTileK);
    a.NS = int(ns);
    a.G = 0;
    // One plan for the whole launch, as for a matrix of all the strips.
    gemv_plan(a.NS, a.KT, dev.cus, &a.WK, &a.SG, &a.RUN, &a.unroll);
    a.DXOK = int64_t(a.NS) * a.SG * a.WK <= 5 * int64_t(dev.cus);
    hipError_t e = launch_gemv_grouped(a, t, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int w2a8_gemv_grouped(int G, const void *const *w_packed, const int64_t *N, int64_t K,
                      const int8_t *x, const float *s_a, const float *s_w,
                      int32_t *const *y_i32, float *const *y_f32, void *workspace,
                      int64_t ws_bytes, void *stream) {
    GemvGroups t;
    int64_t ns = 0, need = 0;
    bool any_f32 = false;
    int st = grouped_setup(G, w_packed, N, K, s_w, y_i32, y_f32, false, &t, &ns, &need, &any_f32);
    if (st != W2A8_OK) return st;
    if (!x || !workspace) return W2A8_ERR_NULL;
    if (any_f32 && !s_a) return W2A8_ERR_NULL;
    if (!aligned(x, 16) || (s_a && !aligned(s_a, 4)) || !aligned(workspace, 16))
        return W2A8_ERR_ALIGN;
    if (ws_bytes < need) return W2A8_ERR_BUFSIZE;
    return grouped_launch(t, ns, K, x, nullptr, s_a, workspace, stream);
}

int w2a8_linear_gemv_grouped(int G, const void *const *w_packed, const int64_t *N, int64_t K,
                             const uint16_t *x_bf16, const float *s_w, float *const *y_f32,
                             int32_t *const *y_i32, void *workspace, int64_t ws_bytes,
                             void *stream) {
    GemvGroups t;
    int64_t ns = 0, need = 0;
    bool any_f32 = false;
    int st = grouped_setup(G, w_packed, N, K, s_w, y_i32, y_f32, true, &t, &ns, &need, &any_f32);
    if (st != W2A8_OK) return st;
    if (!x_bf16 || !workspace) return W2A8_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(workspace, 16)) return W2A8_ERR_ALIGN;
    if (ws_bytes < need) return W2A8_ERR_BUFSIZE;
    return grouped_launch(t, ns, K, nullptr, x_bf16, nullptr, workspace, stream);
}

}  // extern "C"

extern "C" {

// ---------------------------------------------------------------------------
// a8: batched product (device)
// ---------------------------------------------------------------------------
int w2a8_gemm(const void *w_packed, const int8_t *x, int64_t M, int64_t N, int64_t K,
              int32_t *y_i32, const float *s_a, float s_w, float *y_f32, void *workspace,
              int64_t ws_bytes, void *stream) {
    if (!w_packed || !x) return W2A8_ERR_NULL;
    if (!y_i32 && !y_f32) return W2A8_ERR_NULL;
    if (y_f32 && !s_a) return W2A8_ERR_NULL;
    if (!nk_ok(N, K) || M < 1 || M > kMaxM) return W2A8_ERR_SHAPE;
    const int64_t need = w2a8_workspace_bytes(M, N, K);
    if (need > 0 && !workspace) return W2A8_ERR_NULL;
    if (!aligned(w_packed, 16) || !aligned(x, 16) || (y_i32 && !aligned(y_i32, 16)) ||
        (y_f32 && !aligned(y_f32, 16)) || (s_a && !aligned(s_a, 4)) ||
        (workspace && !aligned(workspace, 16)))
        return W2A8_ERR_ALIGN;
    if (ws_bytes < need) return W2A8_ERR_BUFSIZE;
    if (M * round_up(N, kTileRows) > (int64_t(1) << 40)) return W2A8_ERR_SHAPE;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;
    const int64_t Np = round_up(N, kTileRows);
    GemmLaunch a;
    a.wp = static_cast<const uint32_t *>(w_packed);
    a.x = x;
    a.y_i32 = y_i32;
    a.y_f32 = y_f32;
    a.sa = s_a;
    a.sw = s_w;
    a.ws_acc = static_cast<int32_t *>(workspace);
    a.ws_cnt = need > 0 ? reinterpret_cast<uint32_t *>(a.ws_acc + M * Np) : nullptr;
    a.M = int(M);
    a.N = int(N);
    a.K = int(K);
    a.KT = int(round_up(K, kTileK) / kTileK);
    a.NS = int(Np / kTileRows);
    a.shape = gemm_shape(M, N, K, dev.cus, need > 0);
    // Few rows: the GEMV-style kernel over M activation rows.  Automatic
    // choice (measured on MI355X, cold weights): M <= 2 up to 49152 weight
    // tiles (2560 x 6912: 5.1 against 6.7 us for the best MFMA kernel;
    // 5120 x 27648: 10.9 against 14.3 us; at 55296 x 5120 the two tie near
    // 16 us), and ragged K (not a multiple of 16), where the MFMA path is
    // the general kernel.  From M = 3 the MFMA kernels with wave groups
    // splitting K win or tie (5120 x 27648 at M = 4: 14.6 against 16.3 us;
    // 13824 x 2560 at M = 3: 6.2 against 7.2 us).
    const int mode = gemm_kernel_mode();
    const int64_t wtiles = int64_t(a.NS) * a.KT;
    const bool few_auto = K % 16 != 0 || (M <= 2 && wtiles <= 49152);
    const bool few = M <= kRowsMaxM && (mode == 3 || (mode == 0 && few_auto));
    if (few) {
        GemvLaunch g;
        g.wp = a.wp;
        g.x = x;
        g.xb = nullptr;
        g.y_i32 = y_i32;
        g.y_f32 = y_f32;
        g.sa = s_a;
        g.sw = s_w;
        g.ws_row = static_cast<uint64_t *>(workspace);
        g.N = int(N);
        g.K = int(K);
        g.KT = a.KT;
        g.NS = a.NS;
        g.M = int(M);
        g.G = 0;
        gemv_rows_plan(g.NS, g.KT, M, dev.cus, &g.WK, &g.SG, &g.RUN, &g.unroll);
        if (g.SG > 1 && !workspace) return W2A8_ERR_NULL;
        hipError_t e = launch_gemv_rows(g, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
    }
    if (int64_t(a.shape.tiles) + 8 > int64_t(INT32_MAX)) return W2A8_ERR_SHAPE;
    hipError_t e = launch_gemm(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Tuning knobs (w2a8_tuning.h)
// ---------------------------------------------------------------------------
int w2a8_tune_gemv(int wg_per_cu, int tiles_per_wave, int unroll, int krange_tiles,
                   int split_min_tiles) {
    if (wg_per_cu < 1 || wg_per_cu > 64 || tiles_per_wave < 1 || tiles_per_wave > 32 ||
        !(unroll == 2 || unroll == 4 || unroll == 8) || krange_tiles < 1 || krange_tiles > 256 ||
        split_min_tiles < 1)
        return W2A8_ERR_VALUE;
    GemvPolicy &p = gemv_policy();
    p.wg_per_cu = wg_per_cu;
    p.tiles_per_wave = tiles_per_wave;
    p.unroll = unroll;
    p.krange_tiles = krange_tiles;
    p.split_min_tiles = split_min_tiles;
    return W2A8_OK;
}

int w2a8_gemv_plan(int64_t N, int64_t K, int cus, int *waves_per_wg, int *wgs_per_strip,
                   int *unroll, int *stream_waves) {
    if (!waves_per_wg || !wgs_per_strip || !unroll || !stream_waves) return W2A8_ERR_NULL;
    if (!nk_ok(N, K) || cus < 1) return W2A8_ERR_SHAPE;
    const int64_t NS = round_up(N, kTileRows) / kTileRows;
    const int64_t KT = round_up(K, kTileK) / kTileK;
    int run = 0;
    gemv_plan_full(NS, K, cus, waves_per_wg, wgs_per_strip, &run, unroll, stream_waves);
    return W2A8_OK;
}

int w2a8_tune_gemm(int kernel) {
    if (kernel < 0 || kernel > 3) return W2A8_ERR_VALUE;
    gemm_kernel_mode() = kernel;
    return W2A8_OK;
}

int w2a8_tune_gemv_stream(int min_tiles, int waves_per_cu, int unroll) {
    if (min_tiles < 0 || waves_per_cu < 1 || waves_per_cu > 64 ||
        !(unroll == 2 || unroll == 4 || unroll == 8))
        return W2A8_ERR_VALUE;
    GemvPolicy &p = gemv_policy();
    p.stream_min_tiles = min_tiles;
    p.stream_waves_per_cu = waves_per_cu;
    p.stream_unroll = unroll;
    return W2A8_OK;
}

}  // extern "C"
