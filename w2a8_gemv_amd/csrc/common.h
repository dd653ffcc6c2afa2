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
};
GemvPolicy &gemv_policy();

// GEMV launch arguments (passed to the kernel by value).
struct GemvLaunch {
    const uint32_t *wp;
    const int8_t *x;
    int32_t *y_i32;
    float *y_f32;
    const float *sa;
    float sw;
    int32_t *ws_acc;
    uint32_t *ws_cnt;
    int N, K, KT, NS;
    int WK;       // waves per workgroup, splitting its k-range
    int SG;       // workgroups (k-ranges) per row strip
    int RUN;      // longest run of tiles of one wave (<= 32)
    int unroll;
};
// Launch plan for (N, K) on `cus` compute units under the current policy.
void gemv_plan(int64_t NS, int64_t KT, int cus, int *wk, int *sg, int *run, int *unroll);
size_t gemv_lds_bytes(const GemvLaunch &a);
hipError_t launch_gemv(const GemvLaunch &a, hipStream_t stream);

hipError_t launch_quant(const uint16_t *xb, int M, int K, int8_t *xq, float *sa,
                        hipStream_t stream);

// Launch shape of a GEMM: activation rows per workgroup (BM), m- and
// n-blocks (n-block = 4 strips = 128 weight rows), k-parts S, work units.
struct GemmShape {
    int BM, MBLK, NBLK, S, tiles;
};
GemmShape gemm_shape(int64_t M, int64_t N, int64_t K, int cus, bool can_split);

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
