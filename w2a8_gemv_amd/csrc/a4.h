// W2A4 variant: int4 activations in the A4I layout (declarations shared by
// the quantizer, the GEMV and the host entry points).
//
// A4I: a row of K values padded with zeros to Kq = ceil(K/32)*32 values,
// two's complement nibbles, Kq/2 bytes per row.  Value k: chunk c = k/16,
// i = k%16, h = i/4, j = i%4; byte c*8 + 4*(h%2) + j, low nibble for h < 2,
// high nibble otherwise.  So byte j of a chunk's first word holds values j
// and 8+j, byte j of its second word values 4+j and 12+j: the same byte and
// nibble as the codes that the masks 0x33333333 and (w >> 2) & 0x33333333
// select from a T32x128 weight word, which lets v_dot8_i32_i4 pair them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace w2a8 {

constexpr int kA4Granule = 32;   // values per 16-byte granule (row padding unit)

inline int64_t a4_row_bytes(int64_t K) { return (K + kA4Granule - 1) / kA4Granule * 16; }

// Per element (shared by the int4 quantizer kernels and the fused int4
// linear GEMV so all produce the same codes): one correctly rounded fp32
// operation per step, as the int8 quantizer.
// q = clamp(round_half_even(x * inv), -7, 7) as a two's complement nibble.
__device__ __forceinline__ uint32_t q4(float x, float inv) {
    float r = __builtin_rintf(x * inv);
    r = fminf(fmaxf(r, -7.0f), 7.0f);
    return uint32_t(int(r)) & 15u;
}

// Two 32-bit words of one 16-value chunk in the A4I layout: byte j of the
// first word holds values j (low nibble) and 8 + j (high), byte j of the
// second word values 4 + j and 12 + j.
__device__ __forceinline__ void chunk_a4(const float (&v)[16], float inv, uint32_t &w0,
                                         uint32_t &w1) {
    w0 = w1 = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w0 |= (q4(v[j], inv) | (q4(v[8 + j], inv) << 4)) << (8 * j);
        w1 |= (q4(v[4 + j], inv) | (q4(v[12 + j], inv) << 4)) << (8 * j);
    }
}

hipError_t launch_quant_a4(const uint16_t *xb, int M, int K, uint8_t *xq4, float *sa,
                           hipStream_t stream);
// The ring GEMV of gemv_ring.hip with int4 activations (a.x points at the
// A4I row; any K); same plan (gemv_ring_plan), layout, reduction and
// workspace.  depth: 2, 4, 6, 8 or 12 tiles in flight per wave.
hipError_t launch_gemv_a4(const GemvLaunch &a, int depth, hipStream_t stream);
// Its row-slice form (the int8 row-slice kernel's work split: 8 single-wave
// workgroups per strip, each 4 rows of every tile; no split, no workspace),
// for the shapes gemv_slice_plan takes.  depth: 2, 4, 6 or 8 steps of 8 tiles.
hipError_t launch_gemv_a4_slice(const GemvLaunch &a, int depth, hipStream_t stream);
// The same kernel fused with the int4 quantizer (a.xb points at the bf16 row,
// a.x and a.sa unused): every workgroup takes the row maximum and quantizes
// the part of the row its waves consume into LDS.
//  * shared = false: the ring plan's workgroups; each wave's run in its own
//    LDS region (a.RUN <= kA4FusedMaxRun tiles of 64 bytes per wave).
//  * shared = true: a.WK strips per workgroup, one wave each, over one
//    k-range of a.RUN <= kA4SharedMaxRun tiles quantized once into one LDS
//    region; grid x = ceil(NS / a.WK).
hipError_t launch_gemv_a4_fused(const GemvLaunch &a, int depth, bool shared, hipStream_t stream);
constexpr int kA4FusedMaxRun = 64;
constexpr int kA4SharedMaxRun = 1024;

}  // namespace w2a8
