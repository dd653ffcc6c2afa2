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

hipError_t launch_quant_a4(const uint16_t *xb, int M, int K, uint8_t *xq4, float *sa,
                           hipStream_t stream);
// The ring GEMV of gemv_ring.hip with int4 activations (a.x points at the
// A4I row; any K); same plan (gemv_ring_plan), layout, reduction and
// workspace.  depth: 2, 4, 6, 8 or 12 tiles in flight per wave.
hipError_t launch_gemv_a4(const GemvLaunch &a, int depth, hipStream_t stream);

}  // namespace w2a8
