// Fused linear layers on the ring weight stream (bf16 row quantized inside
// the GEMV): the shared launch plan and the int8 launcher (linear_ring.hip).
#pragma once

#include "common.h"

namespace w2a8 {

// Plan of a fused ring kernel, from the ring GEMV's plan (gemv_ring_plan):
// adjusts the launch fields WK, SG and RUN and returns `shared`.
//  * One wave per strip in the ring plan (many strips, or long strips split
//    over workgroups): shared k-ranges.  WS strips per workgroup (one wave
//    each, a->WK = WS) quantize their k-range once; WS = 8 when the strips
//    fill the workgroups (at most 1/32 of the waves idle) and, unsplit,
//    there are at least 1536 strips; otherwise 4.  A split strip with fewer
//    than 200 such workgroups takes twice the k-ranges.  K-ranges hold at
//    most max_shared_run tiles (a->RUN).  Measured on MI355X with the int4
//    kernel (cold, graph of launches, us; WS x k-range factor): 2560 x 6912:
//    8x2 3.88, 8x1 3.97, 4x1 4.67; 5120 x 27648: 8x2 9.99, 4x1 10.32, 8x1
//    11.56; 13824 x 6912: 8x2 6.73, 4x1 7.71; 3200 x 10240 (100 strips):
//    4x1 5.38, 8x1 5.55, 8x2 5.83; 55296 x 5120: 8 13.17, 4 13.78, 16 17.5;
//    20480 x 3200: 4 5.77, 8 7.43, 2 7.77.
//  * Otherwise per-wave runs of at most max_run tiles (a->RUN): more waves
//    (up to 16), then more workgroups per strip, where the ring plan's runs
//    are longer.
// More workgroups per strip than the ring plan's only for split strips or
// for strips longer than 16 * max_run (>= 512) tiles, which exceed every
// k-range bound: the workspace rule of the unfused GEMV still holds.
bool fused_ring_plan(GemvLaunch *a, int max_run, int max_shared_run);

// Kernels of the fused linear layers (values of w2a8_linear_plan's `kernel`).
enum LinearKernel {
    kLinearWorkgroup = 1,   // int8: the workgroup kernel's fused variant (gemv.hip)
    kLinearShared = 3,      // ring kernel over shared k-ranges (WK strips per workgroup)
    kLinearPerWave = 4,     // int4: ring kernel, each wave's run in its own LDS region
};
// The fused layer's launch plan for NS strips of KT tiles: fills a's WK, SG,
// RUN and unroll and returns the kernel.  Int8: the shared ring kernel where
// the ring plan has one wave per strip, else the workgroup kernel (gemv_plan).
// Int4: fused_ring_plan with kA4FusedMaxRun / kA4SharedMaxRun.  *depth: the
// ring depth (ring kernels).
LinearKernel linear_layer_plan(const GemvPolicy &pol, int64_t NS, int64_t KT, int cus, bool int4,
                               GemvLaunch *a, int *depth);

// Int8 fused linear GEMV over shared k-ranges (a plan for which
// fused_ring_plan returned true; a.xb: the bf16 row; a.y_f32 required; a.x,
// a.sa unused; any K).  LDS: a.RUN * 128 bytes, a.RUN <= kLinearSharedMaxRun;
// depth 2, 4, 6, 8 or 12.
constexpr int kLinearSharedMaxRun = 512;
hipError_t launch_linear_ring(const GemvLaunch &a, int depth, hipStream_t stream);

}  // namespace w2a8
