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
// Maximum of a non-negative float over the 64 lanes of a wave, returned
// wave-uniform: four DPP steps inside each row of 16 lanes, then the four
// row maxima read into scalar registers.  Non-negative floats order like
// their bit patterns read as integers.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    int b = __float_as_int(v);
    b = max(b, __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x124, 0xF, 0xF, false));  // row_ror:4
    b = max(b, __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false));  // row_ror:8
    const int r0 = __builtin_amdgcn_readlane(b, 0), r1 = __builtin_amdgcn_readlane(b, 16);
    const int r2 = __builtin_amdgcn_readlane(b, 32), r3 = __builtin_amdgcn_readlane(b, 48);
    return __int_as_float(max(max(r0, r1), max(r2, r3)));
}

__device__ __forceinline__ int sum8(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    return v;
}

// Sum over the 64 lanes of a wave, returned wave-uniform: sum8 and one more
// DPP step give each row of 16 lanes its sum, then the four row sums are
// read into scalar registers.
__device__ __forceinline__ int wave_sum(int v) {
    v = sum8(v);
    v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
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

// The projection a strip belongs to.  Plain launch: the launch's own matrix
// and outputs.  Grouped launch (several projections sharing the activation
// row and K): strips are numbered across the projections in order and
// projection i owns strips [begin[i], begin[i+1]); begin is increasing and
// padded with INT32_MAX, so the choice is a chain of uniform selects over
// values already in the kernel arguments, with no dependent load.
struct Proj {
    const uint32_t *wp;
    int32_t *y_i32;
    float *y_f32;
    float sw;
    int N;
    int s;   // strip index within the projection
};

template <bool GROUPED>
__device__ __forceinline__ Proj select_proj(const GemvLaunch &a, const GemvGroups &t, int s) {
    Proj p{a.wp, a.y_i32, a.y_f32, a.sw, a.N, s};
    if constexpr (GROUPED) {
        // The last projection that begins at or before s owns it.
#pragma unroll
        for (int i = 0; i < kMaxGroups; ++i) {
            const bool hit = s >= t.begin[i];
            p.wp = hit ? t.wp[i] : p.wp;
            p.y_i32 = hit ? t.y_i32[i] : p.y_i32;
            p.y_f32 = hit ? t.y_f32[i] : p.y_f32;
            p.sw = hit ? t.sw[i] : p.sw;
            p.N = hit ? t.N[i] : p.N;
            p.s = hit ? s - t.begin[i] : p.s;
        }
    }
    return p;
}

__device__ __forceinline__ void store_proj(const Proj &p, float sa, int row, int v) {
    if (p.y_i32) p.y_i32[row] = v;
    if (p.y_f32) p.y_f32[row] = (float(v) * sa) * p.sw;
}

}  // namespace w2a8

#endif  // W2A8_DEVICE_H
