// W2A8 GEMV (M = 1) for gfx950.
//
// What it computes — "如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？",
// sections "运行 test.py 做 GEMV 基准测试" and "如何判断结果": y equals the
// exact integer product of int8 activations and ternary weights; with the
// scale epilogue of "Windows 上跑通 BitNet b1.58：…部署实录" §3.1
// (the scale is multiplied back after the integer product).
//
// Design (gfx950, wave64):
//  * Work unit = one wave.  The packed matrix is a sequence of 32-row strips,
//    each a contiguous run of KT 1 KiB tiles.  Strip s is cut into S k-parts;
//    wave (s, p) streams tiles [p*KT/S, (p+1)*KT/S) of strip s, so every wave
//    reads one contiguous byte range with one 16-byte non-temporal load per
//    lane per tile (a whole 1 KiB tile per wave instruction).
//  * Lane l = 8*rg + kg holds rows 4rg..4rg+3 at k = 16kg..16kg+15 of a tile;
//    it loads the matching 16 activation bytes (L1/L2 resident) once and uses
//    them for its four rows.
//  * Decode without sign handling: code c = w + 1 in {0,1,2}.  For a word,
//    the masks 0x03030303, 0x0C0C0C0C, 0x30303030 and (word>>2)&0x30303030
//    leave c, 4c, 16c, 16c in the four bytes, which v_dot4 multiplies with
//    the four activation words; three accumulators (scales 1, 4, 16) are
//    divided back exactly (every partial is a multiple of its scale).  Then
//    sum_k w*x = sum_k c*x - sum_k x, with sum_k x taken once per wave over
//    its k-range.
//  * Reduction: the 8 lanes of a row group are summed with lane shuffles.
//    S == 1: the wave owns the strip and stores y.  S > 1: int32 partials
//    are added atomically into the workspace; the last wave of the strip (an
//    arrival counter) reads the totals, resets workspace and counter, and
//    applies the epilogue.  Integer addition makes the result independent of
//    arrival order, so it is exact and deterministic.
#include "common.h"

namespace w2a8 {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(int(a), int(b), c, false);
}

struct Acc {
    int a1[4], a4[4], a16[4];
};

// One lane slot: 4 rows x 16 k of codes against 16 activation bytes.
__device__ __forceinline__ void mac(const v4u w, const v4u xv, Acc &acc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        acc.a1[q] = dot4(v & 0x03030303u, xv[0], acc.a1[q]);
        acc.a4[q] = dot4(v & 0x0C0C0C0Cu, xv[1], acc.a4[q]);
        acc.a16[q] = dot4(v & 0x30303030u, xv[2], acc.a16[q]);
        acc.a16[q] = dot4((v >> 2) & 0x30303030u, xv[3], acc.a16[q]);
    }
}

// 16 activation bytes at k0..k0+15; bytes at k >= kend read as 0.
__device__ __forceinline__ v4u load_x16(const int8_t *x, int k0, int kend) {
    if (k0 + 16 <= kend) return *reinterpret_cast<const v4u *>(x + k0);
    uint32_t b[4] = {0u, 0u, 0u, 0u};
    for (int i = 0; i < 16; ++i) {
        const int k = k0 + i;
        if (k < kend) b[i >> 2] |= uint32_t(uint8_t(x[k])) << (8 * (i & 3));
    }
    return v4u{b[0], b[1], b[2], b[3]};
}

// sum of x[k0..k1) over the wave (every lane gets the total).
__device__ __forceinline__ int xsum_range(const int8_t *x, int k0, int k1, int lane) {
    int s = 0;
    for (int c = k0 + 16 * lane; c < k1; c += 1024) {
        const v4u v = load_x16(x, c, k1);
        s = dot4(v[0], 0x01010101u, s);
        s = dot4(v[1], 0x01010101u, s);
        s = dot4(v[2], 0x01010101u, s);
        s = dot4(v[3], 0x01010101u, s);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    return s;
}

__device__ __forceinline__ void store_out(const GemvLaunch &a, int row, int v) {
    if (a.y_i32) a.y_i32[row] = v;
    if (a.y_f32) a.y_f32[row] = (float(v) * a.sa[0]) * a.sw;
}

template <int U>
__global__ __launch_bounds__(256) void gemv_kernel(GemvLaunch a) {
    const int lane = threadIdx.x & 63;
    // Wave-uniform values live in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * 4 + (int(threadIdx.x) >> 6));
    if (wave >= a.NS * a.S) return;
    const int s = wave / a.S;
    const int p = wave - s * a.S;
    const int t0 = int((int64_t(p) * a.KT) / a.S);
    const int t1 = int((int64_t(p + 1) * a.KT) / a.S);
    const int kg = lane & 7, rg = lane >> 3;

    const uint32_t *wb = a.wp + int64_t(s) * a.KT * kTileWords + lane * 4;
    const int8_t *xb = a.x + kg * 16;

    Acc acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;

    // Tiles entirely below K need no activation bounds check.
    const int tfull = min(t1, a.K / kTileK);
    int t = t0;
    for (; t + U <= tfull; t += U) {
        v4u w[U], xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            w[u] = __builtin_nontemporal_load(
                reinterpret_cast<const v4u *>(wb + int64_t(t + u) * kTileWords));
#pragma unroll
        for (int u = 0; u < U; ++u)
            xv[u] = *reinterpret_cast<const v4u *>(xb + (t + u) * kTileK);
#pragma unroll
        for (int u = 0; u < U; ++u) mac(w[u], xv[u], acc);
    }
    for (; t < tfull; ++t) {
        const v4u w = __builtin_nontemporal_load(
            reinterpret_cast<const v4u *>(wb + int64_t(t) * kTileWords));
        const v4u xv = *reinterpret_cast<const v4u *>(xb + t * kTileK);
        mac(w, xv, acc);
    }
    // The last tile of a strip may cross K: activations at k >= K read as 0
    // (the packed codes there are 01, weight 0, and do not matter).
    for (; t < t1; ++t) {
        const v4u w = __builtin_nontemporal_load(
            reinterpret_cast<const v4u *>(wb + int64_t(t) * kTileWords));
        const v4u xv = load_x16(a.x, t * kTileK + 16 * kg, a.K);
        mac(w, xv, acc);
    }

    int r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int v = acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4);
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        r[q] = v;
    }
    const int sx = xsum_range(a.x, t0 * kTileK, min(t1 * kTileK, a.K), lane);

    // Lane (rg, kg) with kg < 4 owns row 4rg + kg of the strip.
    const int q = kg & 3;
    const int v = (q == 0 ? r[0] : q == 1 ? r[1] : q == 2 ? r[2] : r[3]) - sx;
    const int row = s * kTileRows + rg * 4 + q;
    const bool owner = kg < 4;

    if (a.S == 1) {
        if (owner && row < a.N) store_out(a, row, v);
        return;
    }
    if (owner)
        __hip_atomic_fetch_add(a.ws_acc + row, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    uint32_t ticket = 0;
    if (lane == 0)
        ticket = __hip_atomic_fetch_add(a.ws_cnt + s, 1u, __ATOMIC_ACQ_REL,
                                        __HIP_MEMORY_SCOPE_AGENT);
    ticket = uint32_t(__shfl(int(ticket), 0));
    if (ticket != uint32_t(a.S - 1)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (owner) {
        const int tot =
            __hip_atomic_exchange(a.ws_acc + row, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (row < a.N) store_out(a, row, tot);
    }
    if (lane == 0)
        __hip_atomic_store(a.ws_cnt + s, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_gemv(const GemvLaunch &a, hipStream_t stream) {
    const int64_t waves = int64_t(a.NS) * a.S;
    const unsigned blocks = unsigned((waves + 3) / 4);
    void *args[] = {const_cast<GemvLaunch *>(&a)};
    const void *fn;
    switch (a.unroll) {
    case 2: fn = reinterpret_cast<const void *>(&gemv_kernel<2>); break;
    case 8: fn = reinterpret_cast<const void *>(&gemv_kernel<8>); break;
    default: fn = reinterpret_cast<const void *>(&gemv_kernel<4>); break;
    }
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, stream);
}

}  // namespace w2a8
