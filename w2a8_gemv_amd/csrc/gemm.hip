// W2A8 batched product (M > 1, prefill) on gfx950 int8 MFMA.
//
// What it computes: the same exact integer product as the GEMV
// ("如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？", sections
// "如何判断结果" and "限制与注意事项" — the reference stops at M == 1), for M
// token rows, Y[m][n] = sum_k X[m][k] * W[n][k], plus the fp32 epilogue.
//
// Design:
//  * v_mfma_i32_16x16x64_i8: A = 16 activation rows x 64 k, B = 64 k x 16
//    weight rows; lane l supplies row (l % 16) and the 16 bytes of k-group
//    (l / 16) of each operand.  A and B use the same lane/byte -> k
//    assignment, so the contraction is exact whatever order the unit sums in.
//  * Workgroup = 4 waves; wave w owns one 32-row weight strip (two 16-row B
//    blocks) and all BM activation rows of the workgroup (BM/16 A blocks).
//  * Weights never go through LDS: a lane loads exactly the packed 32-bit
//    word that holds its B operand (16 codes of one row, 16 consecutive k) and
//    expands it in registers: (word >> 2j) & 0x03030303 gives codes c in
//    bytes, and v_perm_b32 maps c -> c - 1 (0xFF, 0x00, 0x01) in one step.
//  * Activations: one [BM x 128] int8 tile per k-step in LDS (rows padded to
//    144 bytes), double buffered; global loads of the next tile are issued
//    before the MFMAs of the current one.
//  * Work units are (k-part, n-block, m-block) with m fastest; the block id
//    is remapped so that consecutive units land on the same XCD (blocks are
//    dealt round-robin over the 8 XCDs), keeping a weight strip's reuse
//    across m-blocks inside one L2.
//  * Split-K (only when M*N is small): int32 partials are added atomically
//    into the workspace; the last workgroup of a tile (arrival counter)
//    takes the totals, resets them and applies the epilogue.
#include "common.h"

namespace w2a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kXStride = kTileK + 16;  // LDS row stride of the activation tile

struct GemmArgs {
    const uint32_t *wp;
    const int8_t *x;
    int32_t *y_i32;
    float *y_f32;
    const float *sa;
    float sw;
    int32_t *ws_acc;
    uint32_t *ws_cnt;
    int M, N, K, KT, NS, Np;
    int MBLK, NBLK, S, tiles;
};

// Codes {0,1,2} in each byte -> signed weights {-1,0,1}.
__device__ __forceinline__ int signed_codes(uint32_t c) {
    return int(__builtin_amdgcn_perm(0u, 0x000100FFu, c));
}

__device__ __forceinline__ v4i expand_word(uint32_t w) {
    return v4i{signed_codes(w & 0x03030303u), signed_codes((w >> 2) & 0x03030303u),
               signed_codes((w >> 4) & 0x03030303u), signed_codes((w >> 6) & 0x03030303u)};
}

// Load one 16-byte activation chunk (row m, k0..k0+15) with bounds handling.
__device__ __forceinline__ v4u load_x_chunk(const GemmArgs &a, int m, int k0, bool xvec) {
    if (m >= a.M || k0 >= a.K) return v4u{0u, 0u, 0u, 0u};
    const int8_t *p = a.x + int64_t(m) * a.K + k0;
    if (xvec && k0 + 16 <= a.K) return *reinterpret_cast<const v4u *>(p);
    uint32_t b[4] = {0u, 0u, 0u, 0u};
    for (int i = 0; i < 16; ++i)
        if (k0 + i < a.K) b[i >> 2] |= uint32_t(uint8_t(p[i])) << (8 * (i & 3));
    return v4u{b[0], b[1], b[2], b[3]};
}

template <int BM>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
    constexpr int MB = BM / 16;                        // A blocks per wave
    constexpr int XCH = BM * 8;                        // 16-byte chunks per tile
    constexpr int XPT = (XCH + 255) / 256;             // chunks per thread
    __shared__ __attribute__((aligned(16))) int8_t xs[2][BM * kXStride];
    __shared__ uint32_t s_ticket;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int R = int(gridDim.x);  // multiple of 8
    const int unit = (int(blockIdx.x) & 7) * (R >> 3) + (int(blockIdx.x) >> 3);
    if (unit >= a.tiles) return;   // uniform over the workgroup
    const int mb = unit % a.MBLK;
    const int rest = unit / a.MBLK;
    const int nb = rest % a.NBLK;
    const int kp = rest / a.NBLK;
    const int t0 = int(int64_t(kp) * a.KT / a.S), t1 = int(int64_t(kp + 1) * a.KT / a.S);
    const int m0 = mb * BM;
    const int strip = nb * 4 + wv;
    const bool active = strip < a.NS;
    const bool xvec = (a.K & 15) == 0;

    // Word offsets (within a tile) of this lane's four B operands:
    // block j (rows 16j..16j+15 of the strip), k-half h.
    int woff[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 16 * j + (lane & 15);
            const int kg = 4 * h + (lane >> 4);
            woff[j][h] = (8 * (r >> 2) + kg) * 4 + (r & 3);
        }
    const uint32_t *wstrip = a.wp + int64_t(active ? strip : 0) * a.KT * kTileWords;

    v4i acc[MB][2];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // Prologue: activation tile t0 -> LDS buffer 0, weight words of t0.
    v4u xr[XPT];
#pragma unroll
    for (int c = 0; c < XPT; ++c) {
        const int ch = tid + 256 * c;
        if (ch < XCH) xr[c] = load_x_chunk(a, m0 + (ch >> 3), t0 * kTileK + 16 * (ch & 7), xvec);
    }
    uint32_t wcur[2][2] = {{0u, 0u}, {0u, 0u}};
    if (active) {
        const uint32_t *wt = wstrip + int64_t(t0) * kTileWords;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) wcur[j][h] = __builtin_nontemporal_load(wt + woff[j][h]);
    }
#pragma unroll
    for (int c = 0; c < XPT; ++c) {
        const int ch = tid + 256 * c;
        if (ch < XCH)
            *reinterpret_cast<v4u *>(&xs[0][(ch >> 3) * kXStride + 16 * (ch & 7)]) = xr[c];
    }
    __syncthreads();

    int buf = 0;
    for (int t = t0; t < t1; ++t) {
        const bool more = t + 1 < t1;
        // Issue the next tile's loads before this tile's MFMAs.
        uint32_t wnext[2][2] = {{0u, 0u}, {0u, 0u}};
        if (more) {
#pragma unroll
            for (int c = 0; c < XPT; ++c) {
                const int ch = tid + 256 * c;
                if (ch < XCH)
                    xr[c] = load_x_chunk(a, m0 + (ch >> 3), (t + 1) * kTileK + 16 * (ch & 7), xvec);
            }
            if (active) {
                const uint32_t *wt = wstrip + int64_t(t + 1) * kTileWords;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        wnext[j][h] = __builtin_nontemporal_load(wt + woff[j][h]);
            }
        }
        if (active) {
            const int8_t *xt = xs[buf];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const v4i b0 = expand_word(wcur[0][h]);
                const v4i b1 = expand_word(wcur[1][h]);
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const v4i av = *reinterpret_cast<const v4i *>(
                        xt + (16 * i + (lane & 15)) * kXStride + 64 * h + 16 * (lane >> 4));
                    acc[i][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b0, acc[i][0], 0, 0, 0);
                    acc[i][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b1, acc[i][1], 0, 0, 0);
                }
            }
        }
        if (more) {
#pragma unroll
            for (int c = 0; c < XPT; ++c) {
                const int ch = tid + 256 * c;
                if (ch < XCH)
                    *reinterpret_cast<v4u *>(&xs[buf ^ 1][(ch >> 3) * kXStride + 16 * (ch & 7)]) =
                        xr[c];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) wcur[j][h] = wnext[j][h];
        }
        __syncthreads();
        buf ^= 1;
    }

    // Output element of acc[i][j][e]: row m0 + 16i + 4*(lane/16) + e,
    // column strip*32 + 16j + lane%16.
    if (a.S == 1) {
        if (!active) return;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + 16 * i + 4 * (lane >> 4) + e;
                    const int n = strip * kTileRows + 16 * j + (lane & 15);
                    if (m < a.M && n < a.N) {
                        const int v = acc[i][j][e];
                        if (a.y_i32) a.y_i32[int64_t(m) * a.N + n] = v;
                        if (a.y_f32) a.y_f32[int64_t(m) * a.N + n] = (float(v) * a.sa[m]) * a.sw;
                    }
                }
        return;
    }

    if (active) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + 16 * i + 4 * (lane >> 4) + e;
                    const int n = strip * kTileRows + 16 * j + (lane & 15);
                    if (m < a.M)
                        __hip_atomic_fetch_add(a.ws_acc + int64_t(m) * a.Np + n, acc[i][j][e],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
    }
    // All exchanges are device-scope read-modify-write atomics (coherent
    // across the XCDs' L2s); each wave waits for its own to complete before
    // the barrier, so the ticket is taken after every partial sum has landed
    // and no L2 writeback/invalidate fence is needed.
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int cidx = mb * a.NBLK + nb;
    if (tid == 0)
        s_ticket = __hip_atomic_fetch_add(a.ws_cnt + cidx, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket != uint32_t(a.S - 1)) return;
    if (active) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + 16 * i + 4 * (lane >> 4) + e;
                    const int n = strip * kTileRows + 16 * j + (lane & 15);
                    if (m < a.M) {
                        const int v = __hip_atomic_exchange(a.ws_acc + int64_t(m) * a.Np + n, 0,
                                                            __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                        if (n < a.N) {
                            if (a.y_i32) a.y_i32[int64_t(m) * a.N + n] = v;
                            if (a.y_f32)
                                a.y_f32[int64_t(m) * a.N + n] = (float(v) * a.sa[m]) * a.sw;
                        }
                    }
                }
    }
    if (tid == 0)
        __hip_atomic_exchange(a.ws_cnt + cidx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// Shape of a GEMM launch: block rows BM by M, k-split S when few output tiles.
GemmShape gemm_shape(int64_t M, int64_t N, int64_t K, int cus, bool can_split) {
    GemmShape g;
    g.BM = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
    const int64_t NS = round_up(N, kTileRows) / kTileRows;
    const int64_t KT = round_up(K, kTileK) / kTileK;
    g.MBLK = int(ceil_div(M, g.BM));
    g.NBLK = int(ceil_div(NS, 4));
    const int64_t base = int64_t(g.MBLK) * g.NBLK;
    int64_t s = 1;
    if (can_split) {
        s = ceil_div(2 * int64_t(cus), base);
        s = std::min<int64_t>(s, std::max<int64_t>(1, KT / 4));
        s = std::max<int64_t>(1, s);
    }
    g.S = int(s);
    g.tiles = int(base * s);
    return g;
}

hipError_t launch_gemm(const GemmLaunch &l, hipStream_t stream) {
    GemmArgs a;
    a.wp = l.wp;
    a.x = l.x;
    a.y_i32 = l.y_i32;
    a.y_f32 = l.y_f32;
    a.sa = l.sa;
    a.sw = l.sw;
    a.ws_acc = l.ws_acc;
    a.ws_cnt = l.ws_cnt;
    a.M = l.M;
    a.N = l.N;
    a.K = l.K;
    a.KT = l.KT;
    a.NS = l.NS;
    a.Np = l.NS * kTileRows;
    a.MBLK = l.shape.MBLK;
    a.NBLK = l.shape.NBLK;
    a.S = l.shape.S;
    a.tiles = l.shape.tiles;
    const unsigned blocks = unsigned(round_up(a.tiles, 8));
    void *args[] = {&a};
    const void *fn;
    switch (l.shape.BM) {
    case 16: fn = reinterpret_cast<const void *>(&gemm_kernel<16>); break;
    case 32: fn = reinterpret_cast<const void *>(&gemm_kernel<32>); break;
    case 64: fn = reinterpret_cast<const void *>(&gemm_kernel<64>); break;
    default: fn = reinterpret_cast<const void *>(&gemm_kernel<128>); break;
    }
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, stream);
}

}  // namespace w2a8
