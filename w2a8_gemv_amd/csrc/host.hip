// Host side of libw2a8.so: argument validation, the offline steps
// (ternarization and packing) and the device entry points' dispatch.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.h"
#include "knobs.h"
#include "linear_ring.h"
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
        info.lds = int64_t(prop.sharedMemPerBlock);
        g_dev[dev] = info;
        g_dev_status[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? W2A8_OK : W2A8_ERR_ARCH;
        g_dev_known[dev] = true;
    }
    *out = g_dev[dev];
    return g_dev_status[dev];
}

namespace {
std::atomic<int> g_gemm_mode{0};
// Forced plan of the short-batch MFMA ring kernel: waves | depth << 5 |
// workgroups per strip << 9 (0: automatic), one word so that every call
// reads a consistent plan.
std::atomic<uint32_t> g_ring_force{0};
std::mutex g_policy_mu;
GemvPolicy g_policy = {4, 6, 8, 256, 48};

// The forced plan of the current knobs for a strip of KT tiles, if any
// (launch fields WK, SG, RUN, unroll); false for the automatic plan.
bool forced_plan(const GemvPolicy &p, int64_t KT, GemvLaunch *a) {
    if (!p.force_kernel) return false;
    const int64_t SG = std::min<int64_t>(p.force_sg, KT);
    const int64_t ktw = ceil_div(KT, SG);
    const int64_t WK = std::min<int64_t>(p.force_wk, ktw);
    a->SG = int(SG);
    a->WK = int(WK);
    a->RUN = int(ceil_div(ktw, WK));
    a->unroll = p.force_depth;
    return true;
}
}  // namespace

std::atomic<int> g_pipe_force{-1};
int gemm_pipe_force() { return g_pipe_force.load(std::memory_order_relaxed); }
void set_gemm_pipe_force(int cfg) { g_pipe_force.store(cfg, std::memory_order_relaxed); }
int gemm_kernel_mode() { return g_gemm_mode.load(std::memory_order_relaxed); }
void set_gemm_kernel_mode(int mode) { g_gemm_mode.store(mode, std::memory_order_relaxed); }

GemvPolicy gemv_policy() {
    std::lock_guard<std::mutex> lock(g_policy_mu);
    return g_policy;
}

void set_gemv_policy(const GemvPolicy &p) {
    std::lock_guard<std::mutex> lock(g_policy_mu);
    g_policy = p;
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
void gemv_plan(const GemvPolicy &p, int64_t NS, int64_t KT, int cus, int *wk, int *sg, int *run,
               int *unroll) {
    const int64_t tpw = std::max(1, p.tiles_per_wave);
    int64_t SG = ceil_div(KT, std::max(1, p.krange_tiles));
    // (SG > 1 only when gemv_may_split(KT, p): the workspace rule relies on it.)
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


// Short-batch MFMA ring kernel plan (measured on MI355X, cold weights, M = 8
// unless noted; best of sweeps of WK 1..16, SG 1..8, depth 2..8 per shape,
// pipelined kernel in brackets where measured):
//  * at least six strips per CU: one wave per strip, depth 4
//    (55296 x 5120: 15.9 us [16.5]);
//  * three to six strips per CU: two waves per strip, depth 4 (32768 x
//    4096: 9.49 against 10.96 with one wave; 27648 x 5120: 10.20 against
//    10.48 with four waves of depth 2);
//  * K under 40 tiles, or at least 3/4 of a strip per CU: 4 waves per strip,
//    no split, depth 2 for strips of fewer than 32 tiles on at least one
//    strip per CU, else 4 (13824 x 2560: 5.06 us [6.16], M = 4 5.04;
//    20480 x 3200: 6.44, where one wave per strip took 7.90; 6912 x 5120:
//    5.14, where 3 workgroups per strip took 6.04; 2560 x 2560: 3.89;
//    5120 x 3456: 4.39; depth 4 against 2: 8192 x 8192 6.89 against 8.08,
//    8192 x 14336 9.12 against 13.13, 16384 x 8192 9.91 against 10.37);
//  * K of 64 to 127 tiles: 4 waves and 4 workgroups per strip, depth 2
//    (3200 x 10240: 5.77 against 6.29 with 3 workgroups of depth 4);
//  * otherwise 4 waves and 3 workgroups per strip, depth 4 (2 from 128
//    tiles) (2560 x 6912: 4.86 [6.31], M = 4 4.81; 5120 x 27648: 11.2).
// The depth is lowered until the workgroup's rings fit the device's LDS.
void gemm_ring_plan(int64_t NS, int64_t KT, int64_t M, int cus, int64_t lds, int *wk, int *sg,
                    int *depth) {
    int64_t WK = 4, SG = 1, D = 4;
    if (NS >= 6 * int64_t(cus)) {
        WK = 1;
    } else if (NS >= 3 * int64_t(cus)) {
        WK = 2;
    } else if (KT < 40 || 4 * NS >= 3 * int64_t(cus)) {
        D = NS >= cus && KT < 32 ? 2 : 4;
    } else if (KT >= 64 && KT < 128) {
        SG = 4;
        D = 2;
    } else {
        SG = 3;
        D = KT >= 128 ? 2 : 4;
    }
    WK = std::min(WK, ceil_div(KT, SG));
    int d = int(D);
    while (d > 2 && int64_t(gemm_ring_lds_bytes(int(M), int(WK), d)) > lds) d -= 2;
    while (WK > 1 && int64_t(gemm_ring_lds_bytes(int(M), int(WK), d)) > lds) --WK;
    *wk = int(WK);
    *sg = int(SG);
    *depth = d;
}

// Few activation rows: the GEMV plan with runs of at most 8 tiles (one
// activation chunk per lane per row) and at most 32/MR waves per workgroup
// (LDS <= 36 KiB for the MR row regions); more workgroups per strip when
// needed.
void gemv_rows_plan(const GemvPolicy &p, int64_t NS, int64_t KT, int64_t M, int cus, int *wk,
                    int *sg, int *run, int *unroll) {
    int r = 0;
    gemv_plan(p, NS, KT, cus, wk, sg, &r, unroll);
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

}  // namespace w2a8

using namespace w2a8;

extern "C" {

const char *w2a8_status_str(int status) {
    switch (status) {
    case W2A8_OK: return "ok";
    case W2A8_ERR_NULL: return "a required pointer is NULL";
    case W2A8_ERR_SHAPE: return "M, N or K out of range";
    case W2A8_ERR_ALIGN: return "a pointer is not aligned as required";
    case W2A8_ERR_VALUE: return "value out of range (weight, 2-bit code, or tuning knob/forced plan)";
    case W2A8_ERR_BUFSIZE: return "packed or workspace buffer too small";
    case W2A8_ERR_NODEVICE: return "no HIP device available";
    case W2A8_ERR_ARCH: return "current device is not gfx950";
    case W2A8_ERR_LAUNCH: return "kernel launch failed";
    case W2A8_ERR_SCRATCH: return "shape needs more than the static scratch of w2a8_gemv_noalloc";
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
        // GEMV: one 64-bit split-k combining word per padded row, if the
        // plan may split a strip's k-range at all.
        if (gemv_may_split(round_up(K, kTileK) / kTileK, gemv_policy())) bytes = 8 * Np;
    } else if (M <= kRingMaxM) {
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

}  // extern "C"

// Split-k combining words of w2a8_gemv_noalloc: one 64-bit word per padded
// output row, W2A8_NOALLOC_SCRATCH_BYTES in all, one copy per device for the
// life of the process.  Zero when the code object loads; every complete call
// leaves the words it used zero again.  In host code `scratch` names only a
// host-side stand-in: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint64_t scratch[W2A8_NOALLOC_SCRATCH_BYTES / 8];

namespace {

std::mutex g_scratch_mu;
uint64_t *g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

__global__ void clear_words_kernel(uint64_t *p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0;
}

// The device address of `scratch` on device `dev` (current), taken once per
// device.  The first call on a device also clears the array with a fill
// kernel on `stream` (not a memset: callers may be capturing a graph), unless
// the stream is capturing, in which case the load-time zero stands.
int scratch_words(int dev, hipStream_t stream, uint64_t **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return W2A8_ERR_LAUNCH;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return W2A8_ERR_LAUNCH;
        if (cs == hipStreamCaptureStatusNone) {
            hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, stream,
                               static_cast<uint64_t *>(p), int64_t(W2A8_NOALLOC_SCRATCH_BYTES / 8));
            if (hipGetLastError() != hipSuccess) return W2A8_ERR_LAUNCH;
        }
        g_scratch_ptr[dev] = static_cast<uint64_t *>(p);
    }
    *out = g_scratch_ptr[dev];
    return W2A8_OK;
}

}  // namespace

namespace {

// Plans and enqueues one GEMV whose arguments have been validated; `ws` holds
// the split-k combining words (zero on entry and on exit), or is null when
// no plan under `pol` splits a strip.
int gemv_enqueue(const GemvPolicy &pol, const DeviceInfo &dev, const void *w_packed,
                 const int8_t *x, int64_t N, int64_t K, int32_t *y_i32, const float *s_a,
                 float s_w, float *y_f32, uint64_t *ws, void *stream) {
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
    a.ws_row = ws;
    a.N = int(N);
    a.K = int(K);
    a.KT = int(round_up(K, kTileK) / kTileK);
    a.NS = int(Np / kTileRows);
    hipError_t e;
    int depth = 4;
    if (pol.force_kernel == 3) {
        if ((K & 15) != 0) return W2A8_ERR_VALUE;
        a.WK = a.SG = 1;
        a.RUN = a.KT;
        a.unroll = pol.force_depth;
        e = launch_gemv_slice(a, pol.force_depth, static_cast<hipStream_t>(stream));
    } else if (!pol.force_kernel && (K & 15) == 0 && gemv_slice_plan(a.NS, a.KT, dev.cus, &depth)) {
        // few strips, short k-range: 8 row-slice waves per strip, no split
        a.WK = a.SG = 1;
        a.RUN = a.KT;
        a.unroll = depth;
        e = launch_gemv_slice(a, depth, static_cast<hipStream_t>(stream));
    } else if (forced_plan(pol, a.KT, &a)) {
        const hipStream_t st = static_cast<hipStream_t>(stream);
        if (pol.force_kernel == 1) {
            if (a.RUN > 32) return W2A8_ERR_VALUE;
            a.DXOK = pol.force_dx;
            e = launch_gemv(a, st);
        } else {
            if ((K & 15) != 0) return W2A8_ERR_VALUE;
            e = launch_gemv_ring(a, pol.force_depth, st);
        }
    } else if ((K & 15) == 0) {
        gemv_ring_plan(pol, a.NS, a.KT, dev.cus, &a.WK, &a.SG, &a.RUN, &depth);
        a.unroll = depth;
        e = launch_gemv_ring(a, depth, static_cast<hipStream_t>(stream));
    } else {
        // ragged K: the batch kernel (activations staged through LDS)
        gemv_plan(pol, a.NS, a.KT, dev.cus, &a.WK, &a.SG, &a.RUN, &a.unroll);
        a.DXOK = int64_t(a.NS) * a.SG * a.WK <= 5 * int64_t(dev.cus);
        e = launch_gemv(a, static_cast<hipStream_t>(stream));
    }
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------------------
// a4..a7: GEMV (device)
// ---------------------------------------------------------------------------
int w2a8_gemv(const void *w_packed, const int8_t *x, int64_t N, int64_t K, int32_t *y_i32,
              const float *s_a, float s_w, float *y_f32, void *workspace, int64_t ws_bytes,
              void *stream) {
    if (!w_packed || !x) return W2A8_ERR_NULL;
    if (!y_i32 && !y_f32) return W2A8_ERR_NULL;
    if (y_f32 && !s_a) return W2A8_ERR_NULL;
    if (!nk_ok(N, K)) return W2A8_ERR_SHAPE;
    const GemvPolicy pol = gemv_policy();
    const bool need_ws = gemv_may_split(round_up(K, kTileK) / kTileK, pol);
    if (need_ws && !workspace) return W2A8_ERR_NULL;
    if (!aligned(w_packed, 16) || !aligned(x, 16) || (y_i32 && !aligned(y_i32, 16)) ||
        (y_f32 && !aligned(y_f32, 16)) || (s_a && !aligned(s_a, 4)) ||
        (need_ws && !aligned(workspace, 16)))
        return W2A8_ERR_ALIGN;
    if (need_ws && ws_bytes < 8 * round_up(N, kTileRows)) return W2A8_ERR_BUFSIZE;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;

    return gemv_enqueue(pol, dev, w_packed, x, N, K, y_i32, s_a, s_w, y_f32,
                        static_cast<uint64_t *>(workspace), stream);
}

// GEMV with its split-k combining words in the library's static scratch
// array: no workspace argument and no allocation.
int w2a8_gemv_noalloc(const void *w_packed, const int8_t *x, int64_t N, int64_t K,
                      int32_t *y_i32, const float *s_a, float s_w, float *y_f32, void *stream) {
    if (!w_packed || !x) return W2A8_ERR_NULL;
    if (!y_i32 && !y_f32) return W2A8_ERR_NULL;
    if (y_f32 && !s_a) return W2A8_ERR_NULL;
    if (!nk_ok(N, K)) return W2A8_ERR_SHAPE;
    const GemvPolicy pol = gemv_policy();
    const bool need_ws = gemv_may_split(round_up(K, kTileK) / kTileK, pol);
    if (need_ws && 8 * round_up(N, kTileRows) > W2A8_NOALLOC_SCRATCH_BYTES)
        return W2A8_ERR_SCRATCH;
    if (!aligned(w_packed, 16) || !aligned(x, 16) || (y_i32 && !aligned(y_i32, 16)) ||
        (y_f32 && !aligned(y_f32, 16)) || (s_a && !aligned(s_a, 4)))
        return W2A8_ERR_ALIGN;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;
    uint64_t *ws = nullptr;
    if (need_ws) {
        st = scratch_words(dev.id, static_cast<hipStream_t>(stream), &ws);
        if (st != W2A8_OK) return st;
    }
    return gemv_enqueue(pol, dev, w_packed, x, N, K, y_i32, s_a, s_w, y_f32, ws, stream);
}

// Fused linear layer for one token: quant_act_int8 + w2a8_gemv (fp32
// epilogue) in one launch.  Always the workgroup kernel.
int w2a8_linear_gemv(const void *w_packed, const uint16_t *x_bf16, int64_t N, int64_t K, float s_w,
                     float *y_f32, int32_t *y_i32, void *workspace, int64_t ws_bytes,
                     void *stream) {
    if (!w_packed || !x_bf16 || !y_f32) return W2A8_ERR_NULL;
    if (!nk_ok(N, K)) return W2A8_ERR_SHAPE;
    const GemvPolicy pol = gemv_policy();
    const bool need_ws = gemv_may_split(round_up(K, kTileK) / kTileK, pol);
    if (need_ws && !workspace) return W2A8_ERR_NULL;
    if (!aligned(w_packed, 16) || !aligned(x_bf16, 16) || !aligned(y_f32, 16) ||
        (y_i32 && !aligned(y_i32, 16)) || (need_ws && !aligned(workspace, 16)))
        return W2A8_ERR_ALIGN;
    if (need_ws && ws_bytes < 8 * round_up(N, kTileRows)) return W2A8_ERR_BUFSIZE;
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
    // Where the ring plan has one wave per strip (many strips, or long strips
    // split over workgroups): the ring kernel over shared k-ranges; otherwise
    // the workgroup kernel's fused variant.  Measured on MI355X (cold, graph
    // of launches, us; ring / workgroup / quant_act_int8 + w2a8_gemv):
    // 5120 x 27648 10.23 / 18.97 / 15.60; 55296 x 5120 13.46 / 19.03 / 14.96;
    // 2560 x 6912 4.05 / 5.82 / 5.84; 3200 x 10240 5.58 / 7.20 / 7.84;
    // 20480 x 3200 6.33 / 6.80 / 7.30.  With several waves per strip the
    // workgroup kernel wins: 13824 x 2560 5.22 against 5.62 (ring, per-wave
    // runs), 2560 x 2560 3.83 against 3.94.
    int depth = 4;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const hipError_t e =
        linear_layer_plan(pol, a.NS, a.KT, dev.cus, false, &a, &depth) == kLinearShared
            ? launch_linear_ring(a, depth, hs)
            : launch_gemv_fused(a, hs);
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Grouped GEMV: several projections sharing x and K in one launch
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// Validates the projection arrays and fills the table; the launch's NS is
// the total strip count.  `need_f32` makes every y_f32 entry mandatory.
int grouped_setup(const GemvPolicy &pol, int G, const void *const *w_packed, const int64_t *N,
                  int64_t K, const float *s_w, int32_t *const *y_i32, float *const *y_f32,
                  bool need_f32, GemvGroups *t, int64_t *ns_total, int64_t *ws_need,
                  bool *any_f32) {
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
        if (gemv_may_split(round_up(K, kTileK) / kTileK, pol)) ws += 8 * Np;
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

int grouped_launch(const GemvPolicy &pol, const GemvGroups &t, int64_t ns, int64_t K,
                   const int8_t *x, const uint16_t *xb, const float *s_a, void *workspace,
                   void *stream) {
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
    // One plan for the whole launch, as for a matrix of all the strips: the
    // row-slice or ring kernel for int8 rows with K a multiple of 16 (the
    // plain GEMV's rule), else the workgroup kernel (which also quantizes a
    // bf16 row in every workgroup).
    hipError_t e;
    int depth = 4;
    if (!xb && (K & 15) == 0 && gemv_slice_plan(a.NS, a.KT, dev.cus, &depth)) {
        a.WK = a.SG = 1;
        a.RUN = a.KT;
        a.unroll = depth;
        e = launch_gemv_slice_grouped(a, t, depth, static_cast<hipStream_t>(stream));
    } else if (!xb && (K & 15) == 0) {
        gemv_ring_plan(pol, a.NS, a.KT, dev.cus, &a.WK, &a.SG, &a.RUN, &depth);
        a.unroll = depth;
        e = launch_gemv_ring_grouped(a, t, depth, static_cast<hipStream_t>(stream));
    } else {
        gemv_plan(pol, a.NS, a.KT, dev.cus, &a.WK, &a.SG, &a.RUN, &a.unroll);
        a.DXOK = int64_t(a.NS) * a.SG * a.WK <= 5 * int64_t(dev.cus);
        e = launch_gemv_grouped(a, t, static_cast<hipStream_t>(stream));
    }
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
    const GemvPolicy pol = gemv_policy();
    int st = grouped_setup(pol, G, w_packed, N, K, s_w, y_i32, y_f32, false, &t, &ns, &need,
                           &any_f32);
    if (st != W2A8_OK) return st;
    if (!x || (need > 0 && !workspace)) return W2A8_ERR_NULL;
    if (any_f32 && !s_a) return W2A8_ERR_NULL;
    if (!aligned(x, 16) || (s_a && !aligned(s_a, 4)) || (need > 0 && !aligned(workspace, 16)))
        return W2A8_ERR_ALIGN;
    if (ws_bytes < need) return W2A8_ERR_BUFSIZE;
    return grouped_launch(pol, t, ns, K, x, nullptr, s_a, workspace, stream);
}

int w2a8_linear_gemv_grouped(int G, const void *const *w_packed, const int64_t *N, int64_t K,
                             const uint16_t *x_bf16, const float *s_w, float *const *y_f32,
                             int32_t *const *y_i32, void *workspace, int64_t ws_bytes,
                             void *stream) {
    GemvGroups t;
    int64_t ns = 0, need = 0;
    bool any_f32 = false;
    const GemvPolicy pol = gemv_policy();
    int st = grouped_setup(pol, G, w_packed, N, K, s_w, y_i32, y_f32, true, &t, &ns, &need,
                           &any_f32);
    if (st != W2A8_OK) return st;
    if (!x_bf16 || (need > 0 && !workspace)) return W2A8_ERR_NULL;
    if (!aligned(x_bf16, 16) || (need > 0 && !aligned(workspace, 16))) return W2A8_ERR_ALIGN;
    if (ws_bytes < need) return W2A8_ERR_BUFSIZE;
    return grouped_launch(pol, t, ns, K, nullptr, x_bf16, nullptr, workspace, stream);
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
    // Few rows.  Automatic choice (measured on MI355X, cold weights): the
    // dot4 few-row kernel for M <= 2 up to 49152 weight tiles (13824 x 2560
    // at M = 2: 4.92 against 5.07 us for the MFMA ring kernel; 2560 x 6912:
    // 5.1 against 6.7 us for the pipelined kernel) and for ragged K (not a
    // multiple of 16); the MFMA ring kernel for the other M <= 8 (plans
    // above), and for 9 <= M <= 16 with fewer than 3 strips per CU (M = 16
    // against the pipelined kernel: 2560 x 6912 5.89 against 6.61 us,
    // 5120 x 27648 13.4 against 15.6, 3200 x 10240 7.24 against 8.06,
    // 6912 x 5120 6.01 against 6.24, 20480 x 3200 8.20 against 8.45; with
    // more strips the pipelined kernel wins: 27648 x 5120 10.8 against 13.6,
    // 55296 x 5120 17.1 against 18.8); for 17 <= M <= 32 (32-row tiles) only
    // on strips of 192 tiles or more over fewer strips than CUs, where the
    // pipelined kernel reads the weights once per 16-row block (M = 20:
    // 5120 x 27648 16.6 against 19.1 us, 2560 x 27648 12.2 against 14.0; it
    // lost at 112 and 128 tiles: 4096 x 16384 12.0 against 10.0); the
    // pipelined kernel above that.
    const int mode = gemm_kernel_mode();
    const int64_t wtiles = int64_t(a.NS) * a.KT;
    const bool few_auto = K % 16 != 0 || (M <= 2 && wtiles <= 49152);
    const bool few = M <= kRowsMaxM && (mode == 3 || (mode == 0 && few_auto));
    const bool ring_auto = M <= kRowsMaxM ||
                           (M <= kRingAutoMaxM && a.NS < 3 * int64_t(dev.cus)) ||
                           (M <= kRingMaxM && a.KT >= 192 && a.NS < int64_t(dev.cus));
    const bool ring = K % 16 == 0 && !few &&
                      ((mode == 4 && M <= kRingMaxM) || (mode == 0 && ring_auto));
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
        gemv_rows_plan(gemv_policy(), g.NS, g.KT, M, dev.cus, &g.WK, &g.SG, &g.RUN, &g.unroll);
        if (g.SG > 1 && !workspace) return W2A8_ERR_NULL;
        hipError_t e = launch_gemv_rows(g, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
    }
    if (ring) {
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
        int depth = 4;
        const uint32_t f = g_ring_force.load(std::memory_order_relaxed);
        if (f) {
            g.WK = int(f & 31);
            depth = int((f >> 5) & 15);
            g.SG = int(std::min<int64_t>(f >> 9, a.KT));
            if (int64_t(gemm_ring_lds_bytes(int(M), g.WK, depth)) > dev.lds) return W2A8_ERR_VALUE;
        } else {
            gemm_ring_plan(g.NS, g.KT, M, dev.cus, dev.lds, &g.WK, &g.SG, &depth);
        }
        if (g.SG > 1 && !workspace) return W2A8_ERR_NULL;
        hipError_t e = launch_gemm_ring(g, depth, static_cast<hipStream_t>(stream));
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
    GemvPolicy p = gemv_policy();
    p.wg_per_cu = wg_per_cu;
    p.tiles_per_wave = tiles_per_wave;
    p.unroll = unroll;
    p.krange_tiles = krange_tiles;
    p.split_min_tiles = split_min_tiles;
    set_gemv_policy(p);
    return W2A8_OK;
}

int w2a8_tune_gemv_force(int kernel, int waves_per_wg, int wgs_per_strip, int depth,
                         int direct_x) {
    GemvPolicy p = gemv_policy();
    if (kernel == 0) {
        p.force_kernel = p.force_wk = p.force_sg = p.force_depth = p.force_dx = 0;
        set_gemv_policy(p);
        return W2A8_OK;
    }
    if (kernel < 0 || kernel > 3 || waves_per_wg < 1 || waves_per_wg > 16 || wgs_per_strip < 1 ||
        wgs_per_strip > 4096 || (direct_x != 0 && direct_x != 1))
        return W2A8_ERR_VALUE;
    const bool ok = kernel == 1 ? (depth == 2 || depth == 4 || depth == 8) && !(direct_x && depth == 8)
                    : kernel == 2 ? (depth == 2 || depth == 4 || depth == 6 || depth == 8 ||
                                     depth == 12) && direct_x == 1
                                  : (depth == 2 || depth == 4 || depth == 6 || depth == 8) &&
                                        direct_x == 1 && waves_per_wg == 1 && wgs_per_strip == 8;
    if (!ok) return W2A8_ERR_VALUE;
    p.force_kernel = kernel;
    p.force_wk = waves_per_wg;
    p.force_sg = wgs_per_strip;
    p.force_depth = depth;
    p.force_dx = direct_x;
    set_gemv_policy(p);
    return W2A8_OK;
}

int w2a8_gemv_plan(int64_t N, int64_t K, int cus, int *kernel, int *waves_per_wg,
                   int *wgs_per_strip, int *depth) {
    if (!kernel || !waves_per_wg || !wgs_per_strip || !depth) return W2A8_ERR_NULL;
    if (!nk_ok(N, K) || cus < 1) return W2A8_ERR_SHAPE;
    const int64_t NS = round_up(N, kTileRows) / kTileRows;
    const int64_t KT = round_up(K, kTileK) / kTileK;
    int run = 0;
    const GemvPolicy pol = gemv_policy();
    if (K % 16 == 0 && gemv_slice_plan(NS, KT, cus, depth)) {
        *kernel = 3;
        *waves_per_wg = 1;
        *wgs_per_strip = 8;
    } else if (K % 16 == 0) {
        *kernel = 2;
        gemv_ring_plan(pol, NS, KT, cus, waves_per_wg, wgs_per_strip, &run, depth);
    } else {
        *kernel = 1;
        gemv_plan(pol, NS, KT, cus, waves_per_wg, wgs_per_strip, &run, depth);
    }
    return W2A8_OK;
}

int w2a8_linear_plan(int64_t N, int64_t K, int cus, int int4, int *kernel, int *waves_per_wg,
                     int *wgs_per_strip, int *run, int *depth) {
    if (!kernel || !waves_per_wg || !wgs_per_strip || !run || !depth) return W2A8_ERR_NULL;
    if (!nk_ok(N, K) || cus < 1) return W2A8_ERR_SHAPE;
    GemvLaunch a;
    *kernel = linear_layer_plan(gemv_policy(), round_up(N, kTileRows) / kTileRows,
                                round_up(K, kTileK) / kTileK, cus, int4 != 0, &a, depth);
    *waves_per_wg = a.WK;
    *wgs_per_strip = a.SG;
    *run = a.RUN;
    if (*kernel == kLinearWorkgroup) *depth = a.unroll;
    return W2A8_OK;
}

int w2a8_tune_gemm_ring(int waves_per_wg, int wgs_per_strip, int depth) {
    if (waves_per_wg == 0 && wgs_per_strip == 0 && depth == 0) {
        g_ring_force.store(0, std::memory_order_relaxed);
        return W2A8_OK;
    }
    if (waves_per_wg < 1 || waves_per_wg > 16 || wgs_per_strip < 1 || wgs_per_strip > 4096 ||
        !(depth == 2 || depth == 4 || depth == 6 || depth == 8))
        return W2A8_ERR_VALUE;
    g_ring_force.store(uint32_t(waves_per_wg) | uint32_t(depth) << 5 | uint32_t(wgs_per_strip) << 9,
                       std::memory_order_relaxed);
    return W2A8_OK;
}

int w2a8_tune_gemm(int kernel) {
    if (kernel < 0 || kernel > 4) return W2A8_ERR_VALUE;
    set_gemm_kernel_mode(kernel);
    return W2A8_OK;
}

int w2a8_tune_gemm_pipe(int config) {
    if (config < -1 || config >= kGemmPipeConfigs) return W2A8_ERR_VALUE;
    set_gemm_pipe_force(config);
    return W2A8_OK;
}

}  // extern "C"
