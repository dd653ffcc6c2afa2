// Device helpers shared by the kernels (gfx950, wave64).
#ifndef W2A8_DEVICE_H
#define W2A8_DEVICE_H

#include "common.h"

namespace w2a8 {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

// v_dot4_i32_i8: c plus the four products of the signed bytes of a and b.
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(int(a), int(b), c, false);
}

// v_dot8_i32_i4: c plus the eight products of the signed nibbles of a and b
// (nibble i of a with nibble i of b).
__device__ __forceinline__ int dot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8(int(a), int(b), c, false);
}

// Codes {0,1,2} in each byte -> signed weights {-1,0,1} (v_perm_b32 as a
// byte table: selector 0 -> 0xFF, 1 -> 0x00, 2 -> 0x01).
__device__ __forceinline__ int signed_codes(uint32_t c) {
    return int(__builtin_amdgcn_perm(0u, 0x000100FFu, c));
}

// One packed word (16 codes of one weight row at 16 consecutive k) -> the
// 16 signed bytes of an MFMA operand, in k order: the code of k = 4j + b
// sits at bits 8b + 2j, so (word >> 2j) & 0x03030303 holds k = 4j..4j+3 in
// bytes 0..3, the order of the activation bytes in memory.
__device__ __forceinline__ v4i expand_word(uint32_t w) {
    return v4i{signed_codes(w & 0x03030303u), signed_codes((w >> 2) & 0x03030303u),
               signed_codes((w >> 4) & 0x03030303u), signed_codes((w >> 6) & 0x03030303u)};
}

// Sum over the 8 lanes of a row group (lanes 8j..8j+7) with DPP moves:
// xor 1 and xor 2 inside quads, then the mirrored half-row (lane i <-> 7-i).
__device__ __forceinline__ int sum8(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    return v;
}

// Loads of batch b of a wave's run of 1 KiB weight tiles (tiles w0 + b*U + u,
// clamped to the run's last tile `last`): one 16-byte non-temporal load per
// lane per tile.
template <int U>
__device__ __forceinline__ void load_batch(const v4u *wt, int w0, int last, int b, v4u (&w)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        w[u] = __builtin_nontemporal_load(wt + min(w0 + b * U + u, last) * (kTileBytes / 16));
    // Keep the loads here: the scheduler would otherwise sink them towards
    // their uses and shorten the prefetch distance.
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace w2a8

#endif  // W2A8_DEVICE_H
