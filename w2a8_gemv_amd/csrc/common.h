// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "w2a8.h"

namespace w2a8 {

// T32x128 tile geometry (see the layout description in w2a8.h).
constexpr int kTileRows = 32;
constexpr int kTileK = 128;
constexpr int kTileBytes = kTileRows * kTileK / 4;  // 1024
constexpr int kTileWords = kTileBytes / 4;          // 256
constexpr int64_t kMaxN = int64_t(1) << 30;
constexpr int64_t kMaxM = int64_t(1) << 20;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

struct DeviceInfo {
    int id;
    int cus;       // compute units
    int xcds;      // accelerator complex dies sharing the dispatch round robin
    int64_t lds;   // LDS bytes a workgroup may allocate
};

// Queries (once per device) the current device; checks it is gfx950.
int current_device(DeviceInfo *out);

// Launch-shape knobs, settable through w2a8_tuning.h for measurements.
struct GemvPolicy {
    int wg_per_cu;        // workgroups per CU to aim for when strips are split
    int tiles_per_wave;   // target run of 1 KiB tiles per wave
    int unroll;           // largest load batch in tiles (two in flight): 2, 4 or 8
    int krange_tiles;     // at most this many k-tiles per workgroup
    int split_min_tiles;  // split a strip over workgroups only if KT >= this
    // Forced plan for measurement sweeps (force_kernel 0: automatic plan).
    // 1: batch kernel with force_wk waves, force_sg workgroups per strip and
    // load batch force_depth, direct activation loads when force_dx; 2: ring
    // kernel with depth force_depth (activations always loaded directly); 3:
    // row-slice kernel with depth force_depth (force_wk 1, force_sg 8: its
    // 8 slice workgroups per strip, never a k-split).
    int force_kernel = 0, force_wk = 0, force_sg = 0, force_depth = 0, force_dx = 0;
};
// A consistent copy of the current knobs (taken under a lock: every call
// plans from one snapshot, whatever other host threads set meanwhile).
GemvPolicy gemv_policy();
void set_gemv_policy(const GemvPolicy &p);
// True when a GEMV plan under `p` may split a strip of KT tiles over several
// workgroups (and so needs the workspace).  Depends on K alone, not on the
// device.
inline bool gemv_may_split(int64_t KT, const GemvPolicy &p) {
    return KT >= p.split_min_tiles || KT > p.krange_tiles ||
           (p.force_kernel && p.force_kernel != 3 && p.force_sg > 1);
}

// GEMV launch arguments (passed to the kernel by value).
struct GemvLaunch {
    const uint32_t *wp;
    const int8_t *x;
    const uint16_t *xb;   // fused linear GEMV: the bf16 activation row (x unused)
    int32_t *y_i32;
    float *y_f32;
    const float *sa;
    float sw;
    uint64_t *ws_row;   // split-k combining word per padded row (split_word)
    int N, K, KT, NS;
    int M;        // activation rows (the few-row kernel; 1 otherwise)
    int WK;       // waves per workgroup, splitting its k-range
    int SG;       // workgroups (k-ranges) per row strip
    int RUN;      // longest run of tiles of one wave (<= 32)
    int unroll;
    int DXOK = 0; // plain kernel: at most 5 waves per CU in the grid, so activation chunks may
                  // be loaded directly with the weights (latency-bound grids)
    // Workgroup kernel, set by its launcher so that the kernel divides
    // nothing: KT = KQ*SG + KR (k-range g starts at g*KQ + min(g, KR) and has
    // KQ + (g < KR) tiles), and a range of KQ + i tiles = WQi*WK + WRi (wave
    // v starts v*WQi + min(v, WRi) tiles in).
    int KQ, KR, WQ0, WR0, WQ1, WR1;
};
// Grouped GEMV: up to kMaxGroups projections sharing the activation row and K
// in one launch (passed to the kernel by value, next to GemvLaunch, whose NS
// is then the total strip count).  Projection i owns strips [begin[i],
// begin[i+1]); unused entries have begin = INT32_MAX.
constexpr int kMaxGroups = W2A8_MAX_GROUPS;
struct GemvGroups {
    int begin[kMaxGroups];
    int N[kMaxGroups];
    float sw[kMaxGroups];
    const uint32_t *wp[kMaxGroups];
    int32_t *y_i32[kMaxGroups];
    float *y_f32[kMaxGroups];
};
hipError_t launch_gemv_grouped(const GemvLaunch &a, const GemvGroups &t, hipStream_t stream);
// The ring kernel over several projections (K a multiple of 16; gemv_ring.hip).
hipError_t launch_gemv_ring_grouped(const GemvLaunch &a, const GemvGroups &t, int depth,
                                    hipStream_t stream);

// Activation quantization, per element (shared by the quantizer kernel and
// the fused linear GEMV so both produce the same codes): bf16 halves of a
// 32-bit word as fp32, and q = clamp(round_half_even(x * inv), -127, 127)
// as a byte.  Each step is one correctly rounded fp32 operation (the product
// is not contracted: the library is built with -ffp-contract=off).
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t q8(float x, float inv) {
    float r = __builtin_rintf(x * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return uint32_t(uint8_t(int8_t(int(r))));
}

// Split-k combining of a GEMV row with one device-scope atomic per
// contribution.  Each contributor adds (its k-tile count << 40) + its partial
// value to the row's 64-bit word.  The counts reach KT exactly with the last
// contribution, whose returned total then holds the whole row value
// (|value| <= K*127 < 2^27, far from the count field); that contributor
// stores the row and clears the word.  Integer addition makes the result
// independent of arrival order, and no ticket or fence is needed.
constexpr int kCountShift = 40;
__device__ __forceinline__ uint64_t split_word(int tiles, int val) {
    return (uint64_t(uint32_t(tiles)) << kCountShift) + uint64_t(int64_t(val));
}
// Given the word's total after adding a contribution: true (with the row
// value in *v, and the word cleared) when it was the last one.
__device__ __forceinline__ bool split_done(uint64_t *word, uint64_t tot, int kt, int *v) {
    const uint64_t cnt = (tot + (uint64_t(1) << (kCountShift - 1))) >> kCountShift;
    if (cnt != uint64_t(uint32_t(kt))) return false;
    *v = int(int64_t(tot - (uint64_t(uint32_t(kt)) << kCountShift)));
    __hip_atomic_store(word, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}
// Adds a contribution of `tiles` k-tiles; true (row value in *v) for the last.
__device__ __forceinline__ bool split_add(uint64_t *word, int tiles, int val, int kt, int *v) {
    const uint64_t add = split_word(tiles, val);
    return split_done(
        word, __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add,
        kt, v);
}

// Launch plan for (N, K) on `cus` compute units under policy `p`.
void gemv_plan(const GemvPolicy &p, int64_t NS, int64_t KT, int cus, int *wk, int *sg, int *run,
               int *unroll);
size_t gemv_lds_bytes(const GemvLaunch &a);
// Ring-kernel plan of the plain GEMV (K a multiple of 16).
void gemv_ring_plan(const GemvPolicy &p, int64_t NS, int64_t KT, int cus, int *wk, int *sg,
                    int *run, int *depth);
// Few activation rows (2 <= M <= 8): plan with runs of at most 8 tiles, and
// the kernel (gemv.hip).  Workspace: 8 bytes per (row, padded output) when
// strips are split.
void gemv_rows_plan(const GemvPolicy &p, int64_t NS, int64_t KT, int64_t M, int cus, int *wk,
                    int *sg, int *run, int *unroll);
hipError_t launch_gemv_rows(const GemvLaunch &a, hipStream_t stream);
constexpr int64_t kRowsMaxM = 8;
// Short batches on MFMA (gemm_ring.hip): 2 <= M <= kRingMaxM, K a multiple
// of 16, the GEMV's work split (WK waves, SG workgroups per strip; split
// strips combine per (row, output) like the few-row kernel), depth 2, 4, 6
// or 8 tiles in flight per wave, activation tiles of 8, 16 or 32 rows.  LDS:
// gemm_ring_lds_bytes per workgroup.  The automatic choice takes it up to
// kRingAutoMaxM rows, and up to kRingMaxM rows on very long strips.
constexpr int64_t kRingMaxM = 32;
constexpr int64_t kRingAutoMaxM = 16;
size_t gemm_ring_lds_bytes(int M, int wk, int depth);
hipError_t launch_gemm_ring(const GemvLaunch &a, int depth, hipStream_t stream);
// Fused linear GEMV: quantize the bf16 row in every workgroup, then the
// workgroup kernel with the fp32 epilogue (gemv.hip).
hipError_t launch_gemv_fused(const GemvLaunch &a, hipStream_t stream);
hipError_t launch_gemv(const GemvLaunch &a, hipStream_t stream);
// Ring-pipelined GEMV (gemv_ring.hip): K a multiple of 16, WK <= 16 waves
// per workgroup, depth 2, 4, 6, 8 or 12 tiles in flight per wave.
hipError_t launch_gemv_ring(const GemvLaunch &a, int depth, hipStream_t stream);
// Row-slice GEMV (gemv_ring.hip): K a multiple of 16, 8 single-wave
// workgroups per strip (each 4 rows of every tile), no split, no workspace;
// depth 2, 4, 6 or 8 steps of 8 tiles in flight per wave.  The plan returns
// true (with the depth) for the shapes it serves by default.
bool gemv_slice_plan(int64_t NS, int64_t KT, int cus, int *depth);
hipError_t launch_gemv_slice(const GemvLaunch &a, int depth, hipStream_t stream);
// The row-slice kernel over several projections (strips numbered across them).
hipError_t launch_gemv_slice_grouped(const GemvLaunch &a, const GemvGroups &t, int depth,
                                     hipStream_t stream);

hipError_t launch_quant(const uint16_t *xb, int M, int K, int8_t *xq, float *sa,
                        hipStream_t stream);

// Launch shape of a GEMM: activation rows per workgroup (BM), m- and
// n-blocks (n-block = 4 strips = 128 weight rows), k-parts S, work units.
struct GemmShape {
    int BM, MBLK, NBLK, S, tiles;
    int pipe;   // pipelined-kernel configuration, or -1 for the general kernel
};
GemmShape gemm_shape(int64_t M, int64_t N, int64_t K, int cus, bool can_split);
// Kernel choice knob (w2a8_tune_gemm): 0 automatic, 1 pipelined kernel
// whenever K allows it, 2 general kernel always, 3 few-row GEMV-style kernel
// whenever M <= 8.  Modes 1 and 2 never pick the few-row kernel.  Read and
// set atomically.
int gemm_kernel_mode();
void set_gemm_kernel_mode(int mode);

// Split-K is only ever used when M * Np <= kGemmSplitMaxOut, which bounds the
// workspace that w2a8_workspace_bytes reports.
constexpr int64_t kGemmSplitMaxOut = int64_t(1) << 22;

struct GemmLaunch {
    const uint32_t *wp;
    const int8_t *x;
    int32_t *y_i32;
    float *y_f32;
    const float *sa;
    float sw;
    int32_t *ws_acc;
    uint32_t *ws_cnt;
    int M, N, K, KT, NS;
    GemmShape shape;
};
hipError_t launch_gemm(const GemmLaunch &a, hipStream_t stream);

}  // namespace w2a8
