// W2A8 batched product (M > 1, prefill) on gfx950 int8 MFMA.
//
// What it computes: the same exact integer product as the GEMV
// ("如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？", sections
// "如何判断结果" and "限制与注意事项" — the reference stops at M == 1), for M
// token rows, Y[m][n] = sum_k X[m][k] * W[n][k], plus the fp32 epilogue.
//
// Both kernels use v_mfma_i32_16x16x64_i8: A = 16 activation rows x 64 k,
// B = 64 k x 16 weight rows; lane l supplies row (l % 16) and the 16 bytes of
// k-group (l / 16) of each operand.  A and B use the same lane/byte -> k
// assignment, so the contraction is exact whatever order the unit sums in.
// Weight codes are expanded in registers: (word >> 2j) & 0x03030303 gives
// codes c in bytes, and v_perm_b32 maps c -> c - 1 (0xFF, 0x00, 0x01).
//
// The pipelined kernel (gemm_pipe_kernel, below) serves K a multiple of 16:
// both operands stream through a ring of LDS stages by direct global->LDS
// loads, several k-tiles ahead.  The general kernel serves every shape and
// adds split-K for small outputs:
//  * Workgroup = 4 waves; wave w owns one 32-row weight strip (two 16-row B
//    blocks) and all BM activation rows of the workgroup (BM/16 A blocks).
//  * Weights never go through LDS: a lane loads exactly the packed 32-bit
//    word that holds its B operand (16 codes of one row, 16 consecutive k).
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
#include "knobs.h"
#include "device.h"

namespace w2a8 {
namespace {

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
    // Set by the launcher so that the kernel divides nothing: KT = KQ*S + KR
    // (k-part p starts at p*KQ + min(p, KR)).
    int KQ, KR;
};

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
    // Work unit (m-block fastest, then n-block, then k-part), remapped from
    // the block id so that consecutive units land on one XCD.
    const int R = int(gridDim.x);  // multiple of 8
    const int unit = (int(blockIdx.x) & 7) * (R >> 3) + (int(blockIdx.x) >> 3);
    if (unit >= a.tiles) return;   // uniform over the workgroup
    const int mb = unit % a.MBLK;
    const int rest = unit / a.MBLK;
    const int nb = rest % a.NBLK;
    const int kp = rest / a.NBLK;
    const int t0 = kp * a.KQ + min(kp, a.KR);
    const int t1 = t0 + a.KQ + (kp < a.KR ? 1 : 0);
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

template <int BM, int WM, int WN, int SPW, int S>
struct Pipe {
    static constexpr int NW = WM * WN;
    static constexpr int MBW = BM / WM / 16;           // A blocks per wave
    static constexpr int NBW = 2 * SPW;                // B blocks per wave
    static constexpr int NSTRIP = WN * SPW;            // strips per workgroup
    static_assert(NSTRIP % NW == 0, "whole weight strips per wave");
    static constexpr int LS = NSTRIP / NW;             // weight strip loads per wave per tile
    // The activation tile is NPART parts of 1 KiB (one load instruction
    // each).  With fewer parts than waves (16-row tiles), waves w and
    // w + NPART load the same part: every wave then issues the same number of
    // loads, so the wait counts below stay compile-time constants.
    static constexpr int NPART = BM * 8 / 64;
    static constexpr int DPW = NPART >= NW ? NPART / NW : 1;   // activation loads per wave per tile
    static_assert(NPART >= NW ? DPW * NW == NPART : NW % NPART == 0,
                  "tile must split evenly over waves");
    // Part loaded by instruction d of wave wv.
    static __device__ __forceinline__ int part(int wv, int d) {
        return NPART >= NW ? wv * DPW + d : wv % NPART;
    }
    static constexpr int LPT = DPW + LS;               // loads per wave per tile
    static constexpr int WAITN = (S - 2) * LPT;        // issued after a tile's group when used
    static_assert(WAITN <= 63, "wait count must fit vmcnt");
    static constexpr int XBYTES = BM * kTileK;
    static constexpr int STAGE = XBYTES + NSTRIP * kTileBytes;
};

// Loads of k-tile tc into one group's part of a ring stage: this wave's DPW
// activation instructions and its LS weight strips.
template <int BM, int WM, int WN, int SPW, int S>
__device__ __forceinline__ void pipe_issue(int8_t *stage, int tc, int K, int wv,
                                           const int8_t *const *xsrc, const int *kcb,
                                           const int8_t *const *wsrc) {
    using P = Pipe<BM, WM, WN, SPW, S>;
#pragma unroll
    for (int d = 0; d < P::DPW; ++d) {
        const int k0 = tc * kTileK + kcb[d];
        const int k = k0 < K - 16 ? k0 : K - 16;
        __builtin_amdgcn_global_load_lds(
            xsrc[d] + k,
            (__attribute__((address_space(3))) void *)(stage + P::part(wv, d) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int ls = 0; ls < P::LS; ++ls)
        __builtin_amdgcn_global_load_lds(
            wsrc[ls] + int64_t(tc) * kTileBytes,
            (__attribute__((address_space(3))) void *)(stage + P::XBYTES +
                                                        (wv * P::LS + ls) * kTileBytes),
            16, 0, 0);
}

// MFMAs of the tile in ring stage s.
template <int BM, int WM, int WN, int SPW, int S>
__device__ __forceinline__ void pipe_mma(const int8_t *stage,
                                         const int (&aoff)[Pipe<BM, WM, WN, SPW, S>::MBW][2],
                                         const int (&boff)[Pipe<BM, WM, WN, SPW, S>::NBW][2],
                                         v4i (&acc)[Pipe<BM, WM, WN, SPW, S>::MBW]
                                                   [Pipe<BM, WM, WN, SPW, S>::NBW]) {
    using P = Pipe<BM, WM, WN, SPW, S>;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        v4i bf[P::NBW];
#pragma unroll
        for (int j = 0; j < P::NBW; ++j)
            bf[j] = expand_word(*reinterpret_cast<const uint32_t *>(stage + boff[j][h]));
#pragma unroll
        for (int i = 0; i < P::MBW; ++i) {
            const v4i av = *reinterpret_cast<const v4i *>(stage + aoff[i][h]);
#pragma unroll
            for (int j = 0; j < P::NBW; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bf[j], acc[i][j], 0, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel (K a multiple of 16).
//
//  * Workgroup = WM x WN waves; wave (wm, wn) owns rows m0 + wm*BM/WM ..
//    (BM/WM rows, MBW A blocks) and SPW consecutive 32-row weight strips
//    (NBW = 2*SPW B blocks).  Workgroup tile: BM rows x WN*SPW strips.
//  * Both operands reach LDS by direct global->LDS loads (global_load_lds,
//    16 bytes per lane, 1 KiB per wave instruction) into a ring of S
//    stages, so S-1 k-tiles are in flight with no register staging.  A stage
//    holds the [BM x 128] activation tile, 16-byte chunk (r, c) at position
//    8r + (c ^ (r & 7)) (row loads stay 128-byte coalesced, A fragment reads
//    of 16 rows at one chunk spread over the banks), then the packed 1 KiB
//    tile of each of the workgroup's strips with its 16-byte slots permuted
//    (XOR within groups of 8) so that B operand reads are conflict-free.
//  * Each lane reads the four packed words of its B operands from LDS and
//    expands them in registers (codes -> {-1, 0, 1} with v_perm_b32).
//  * Per k-tile: wait for this wave's loads of the tile (the compiler does not
//    track global->LDS loads: the count is explicit), barrier, refill the
//    stage freed by the previous tile, then the MFMAs.
//  * Rows past M read row M-1 and k-chunks past K read a chunk inside the
//    row: their products reach only discarded outputs or meet the weight
//    padding (code 01, weight 0).  Strips past the matrix read its last strip.
//  * KS > 1 (small output grids, where one wave's k-step latency is the
//    bound): KS groups of WM x WN waves split the k-range inside the
//    workgroup, group g taking k-tiles g, g + KS, ...; each ring stage holds
//    one part per group, all groups step together, and at the end groups
//    1..KS-1 hand their accumulators to group 0 through LDS.
template <int BM, int WM, int WN, int SPW, int S, int KS>
__global__ __launch_bounds__(64 * WM * WN * KS) void gemm_pipe_kernel(GemmArgs a) {
    using P = Pipe<BM, WM, WN, SPW, S>;
    constexpr int MBW = P::MBW, NBW = P::NBW, DPW = P::DPW, WAITN = P::WAITN;
    constexpr int GS = P::STAGE, SS = KS * P::STAGE;   // group part, whole stage
    static_assert((KS - 1) * P::NW * MBW * NBW * 4 * 64 * 4 <= S * SS,
                  "group reduction must fit in the ring");
    __shared__ __attribute__((aligned(1024))) int8_t ring[S * SS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wvall = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wvall / P::NW;                 // k-group
    const int wv = wvall - grp * P::NW;            // wave within the group
    const int wm = wv / WN, wn = wv - (wv / WN) * WN;
    const int R = int(gridDim.x);  // multiple of 8
    const int unit = (int(blockIdx.x) & 7) * (R >> 3) + (int(blockIdx.x) >> 3);
    if (unit >= a.tiles) return;   // uniform over the workgroup
    const int mb = unit % a.MBLK;
    const int nb = unit / a.MBLK;
    const int m0 = mb * BM;
    const int KT = a.KT;

    // Activation loads: instruction d of this wave covers chunk positions
    // p = part(wv, d)*64 + lane of a stage.
    const int8_t *xsrc[P::DPW];
    int kcb[P::DPW];
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
        const int p = P::part(wv, d) * 64 + lane;
        const int r = p >> 3, c = (p & 7) ^ (r & 7);
        xsrc[d] = a.x + int64_t(min(m0 + r, a.M - 1)) * a.K;
        kcb[d] = 16 * c;
    }
    // Weight loads: this wave brings strips wv*LS .. wv*LS+LS-1 of the
    // workgroup.  Lane l loads 16-byte slot 8(l>>3) + ((l & 7) ^ 2((l>>3) & 3))
    // of the tile into LDS position l (an XOR within each group of 8 slots,
    // its own inverse), so that the B operand reads below hit 32 distinct
    // banks.
    const int wslot = 8 * (lane >> 3) + ((lane & 7) ^ (2 * ((lane >> 3) & 3)));
    const int8_t *wsrc[P::LS];
#pragma unroll
    for (int ls = 0; ls < P::LS; ++ls) {
        const int sload = min(nb * P::NSTRIP + wv * P::LS + ls, a.NS - 1);
        wsrc[ls] = reinterpret_cast<const int8_t *>(a.wp) + int64_t(sload) * KT * kTileBytes +
                   16 * wslot;
    }

    v4i acc[MBW][NBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // A fragment byte offsets within a stage, per block i and k-half h.
    int aoff[MBW][2];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = wm * (BM / WM) + 16 * i + (lane & 15);
            const int c = 4 * h + (lane >> 4);
            aoff[i][h] = (r * 8 + (c ^ (r & 7))) * 16;
        }
    // B operand word offsets (bytes) within a stage: strip sp of the wave,
    // rows 16jb..16jb+15 of it, k-half h.
    int boff[NBW][2];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 16 * jb + (lane & 15);
                const int kg = 4 * h + (lane >> 4);
                const int g = r >> 2;                    // slot 8g + kg, stored at
                const int pos = 8 * g + (kg ^ (2 * (g & 3)));   // position pos
                boff[2 * sp + jb][h] = P::XBYTES + (wn * SPW + sp) * kTileBytes +
                                       (pos * 4 + (r & 3)) * 4;
            }

    // Group grp's k-tile of step tt (past the last: a repeat of it, loaded
    // to keep the wait counts exact, never multiplied).
    const int nsteps = (KT + KS - 1) / KS;
#define W2A8_PIPE_TILE(tt) min((tt) * KS + grp, KT - 1)
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
        pipe_issue<BM, WM, WN, SPW, S>(ring + s * SS + grp * GS, W2A8_PIPE_TILE(s), a.K, wv, xsrc,
                                       kcb, wsrc);

    // One k-tile: this wave's loads of the tile have landed and its LDS reads
    // of the previous tile are done (lgkmcnt 0); after the barrier that holds
    // for every wave.  A plain s_barrier: a fence here would wait for every
    // load in flight; the empty asm keeps the compiler from moving memory
    // accesses across it.  Then refill the stage the previous tile used
    // (past the last tile: a repeat of it, never used, which keeps the wait
    // count exact) and multiply.
#define W2A8_PIPE_STEP(s, tt)                                                                    \
    do {                                                                                         \
        __builtin_amdgcn_s_waitcnt((WAITN & 15) | ((WAITN >> 4) << 14) | (0x7 << 4));            \
        __builtin_amdgcn_s_barrier();                                                            \
        __asm__ volatile("" ::: "memory");                                                       \
        pipe_issue<BM, WM, WN, SPW, S>(ring + (((s) + S - 1) % S) * SS + grp * GS,               \
                                       W2A8_PIPE_TILE((tt) + S - 1), a.K, wv, xsrc, kcb, wsrc);  \
        if (KS == 1 || (tt) * KS + grp < KT)                                                     \
            pipe_mma<BM, WM, WN, SPW, S>(ring + (s) * SS + grp * GS, aoff, boff, acc);           \
    } while (0)

    // Whole groups of S steps, then the remainder.
    int t = 0;
    for (; t + S <= nsteps; t += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) W2A8_PIPE_STEP(s, t + s);
    }
    const int rem = nsteps - t;
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
        if (s < rem) W2A8_PIPE_STEP(s, t + s);
#undef W2A8_PIPE_STEP
#undef W2A8_PIPE_TILE

    if constexpr (KS > 1) {
        // Every load in flight has landed and every LDS read is done once all
        // waves pass this fence-and-barrier; the ring is then free.
        __syncthreads();
        int *red = reinterpret_cast<int *>(ring);
        if (grp > 0) {
#pragma unroll
            for (int i = 0; i < MBW; ++i)
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        red[((((grp - 1) * P::NW + wv) * MBW + i) * NBW * 4 + j * 4 + e) * 64 + lane] =
                            acc[i][j][e];
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int q = 1; q < KS; ++q)
#pragma unroll
            for (int i = 0; i < MBW; ++i)
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j][e] +=
                            red[((((q - 1) * P::NW + wv) * MBW + i) * NBW * 4 + j * 4 + e) * 64 + lane];
    }

    // Output element of acc[i][j][e]: row m0 + wm*BM/WM + 16i + 4*(lane/16) + e,
    // column strip(j/2)*32 + 16*(j%2) + lane%16.  Activation scales of this
    // lane's rows are all loaded before any store (a wait between stores would
    // also wait for the stores before it).
    float sa[MBW][4] = {};
    if (a.y_f32) {
#pragma unroll
        for (int i = 0; i < MBW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sa[i][e] = a.sa[min(m0 + wm * (BM / WM) + 16 * i + 4 * (lane >> 4) + e, a.M - 1)];
        __builtin_amdgcn_s_waitcnt(0x0070 | (0xF << 8));   // vmcnt(0)
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int strip = nb * P::NSTRIP + wn * SPW + j / 2;
        const int n = strip * kTileRows + 16 * (j & 1) + (lane & 15);
        if (strip >= a.NS || n >= a.N) continue;
#pragma unroll
        for (int i = 0; i < MBW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * (BM / WM) + 16 * i + 4 * (lane >> 4) + e;
                if (m < a.M) {
                    const int v = acc[i][j][e];
                    if (a.y_i32) a.y_i32[int64_t(m) * a.N + n] = v;
                    if (a.y_f32) a.y_f32[int64_t(m) * a.N + n] = (float(v) * sa[i][e]) * a.sw;
                }
            }
    }
}

}  // namespace

// Shape of a GEMM launch: block rows BM by M, k-split S when few output tiles.
// Pipelined-kernel configurations: (BM, WM, WN, SPW, ring depth, wave groups
// splitting K).  Chosen by sweeps on MI355X over block rows 32..256, four
// wave layouts, depths 3..8 and 1, 2 or 4 wave groups: 32 rows (depth 4) for
// M <= 32 and 64 rows (depth 3) above won or tied on every prefill shape with
// a large output grid up to M = 448, a 128 x 256 tile beyond, 32 rows (16
// for M <= 16) with 2 or 4 wave groups (depth 3) on small grids, and
// workgroups of 1 or 2 strips with 4 or 8 wave groups on the smallest grids
// with K of 20 tiles or more.
struct PipeCfg {
    int BM, WM, WN, SPW, S, KS;
};
constexpr PipeCfg kPipeCfg[10] = {{32, 1, 4, 1, 4, 1}, {64, 1, 4, 1, 3, 1}, {128, 1, 8, 1, 4, 1},
                                  {32, 1, 4, 1, 3, 2}, {32, 1, 4, 1, 3, 4}, {16, 1, 4, 1, 3, 2},
                                  {16, 1, 4, 1, 3, 4}, {32, 1, 2, 1, 3, 4}, {16, 1, 2, 1, 3, 8},
                                  {16, 1, 1, 1, 3, 8}};

// The kernel instance of configuration P.
template <int P>
const void *pipe_kernel_fn() {
    constexpr PipeCfg c = kPipeCfg[P];
    return reinterpret_cast<const void *>(&gemm_pipe_kernel<c.BM, c.WM, c.WN, c.SPW, c.S, c.KS>);
}

GemmShape gemm_shape(int64_t M, int64_t N, int64_t K, int cus, bool can_split) {
    GemmShape g;
    g.pipe = -1;
    if (K >= 16 && K % 16 == 0) {
        // Pipelined kernel (measured on MI355X, cold weights):
        //  * small output grids (at most 7/4 workgroups of 32 rows x 4 strips
        //    per CU, K of 8 tiles or more): 32-row tiles with the k-range split
        //    over wave groups inside the workgroup, 4 groups when the grid is
        //    at most one per CU and K has 40 tiles or more, else 2 (the lone
        //    wave's k-step latency is the bound there: 2560 x 6912 at M = 128
        //    went from 22.4 to 12.6 us, 13824 x 2560 at M = 8 from 9.3 to
        //    7.3 us); 16-row tiles for M <= 16, whose activation tile is
        //    half as large (55296 x 5120 at M = 8: 15.2 against 16.9 us);
        //    For M > 32 that holds up to 2 such workgroups per CU (a sweep of
        //    every configuration off the workload shapes: 4096 x 4096 at
        //    M = 512 14.9 against 19.2 us with 64-row tiles, 8192 x 8192 at
        //    M = 256 26.2 against 33.3, 16384 x 4096 at M = 128 15.4
        //    against 19.4);
        //  * otherwise 32 or 64 rows per workgroup by M, and a 128 x 256
        //    workgroup tile (8 waves, each decoded weight block used by 8
        //    activation blocks) for M > 128 over more than 4 such 32-row
        //    workgroups per CU (24.7 against 29.9 us at M = 512,
        //    13824 x 2560; 31.4 against 41.9 at M = 256, 28672 x 4096; at
        //    4 per CU the 64-row tile is still ahead: 8192 x 8192 at
        //    M = 512 40.7 against 49.9, 16384 x 4096 at M = 256 23.3
        //    against 29.1);
        //  * K of 20 tiles or more over few strips: workgroups of one strip
        //    with 8 wave groups and 16-row tiles while that grid is at most
        //    one workgroup per CU (2560 x 6912 at M = 8: 6.0 against 8.2 us,
        //    5120 x 27648 at M = 8: 14.6 against 18.2 us), else workgroups
        //    of 2 strips, so that the grid doubles, with 8 wave groups and
        //    16-row tiles while that grid is, else 4 groups and 32-row tiles
        //    while that one is (2560 x 6912 at M = 64: 8.0 against 13.1 us,
        //    at M = 128: 9.6 against 12.6 us; 5120 x 27648 at M = 32: 18.6
        //    against 31 us; 13824 x 2560 at M = 8: 6.1 against 7.2 us).
        //    These also beat the general kernel's split over K across
        //    workgroups on every grid it used to take (at most one 32-row
        //    workgroup per 4 CUs with 96 k-tiles or more: 5120 x 27648 at
        //    M = 8, 14.6 against 23.6 us), so the automatic choice no longer
        //    takes it when K is a multiple of 16.
        const int64_t NS = round_up(N, kTileRows) / kTileRows;
        const int64_t KT = round_up(K, kTileK) / kTileK;
        const int64_t g32 = ceil_div(M, 32) * ceil_div(NS, 4);
        const int64_t n2 = ceil_div(NS, 2);
        const bool narrow = KT >= 20;
        const bool one16 = narrow && ceil_div(M, 16) * NS <= cus;
        const bool narrow16 = narrow && ceil_div(M, 16) * n2 <= cus;
        const bool narrow32 = narrow && ceil_div(M, 32) * n2 <= cus;
        int pipe;
        if (gemm_pipe_force() >= 0)
            pipe = gemm_pipe_force();
        else if (one16)
            pipe = 9;
        else if (narrow16)
            pipe = 8;
        else if (narrow32)
            pipe = 7;
        else if (KT >= 8 && (g32 <= int64_t(cus) * 7 / 4 || (M > 32 && g32 <= 2 * int64_t(cus))))
            pipe = ((KT >= 40 && g32 <= cus) ? 4 : 3) + (M <= 16 ? 2 : 0);
        else
            pipe = M <= 32 ? 0 : (M > 128 && g32 > 4 * int64_t(cus)) ? 2 : 1;
        const PipeCfg &c = kPipeCfg[pipe];
        const int64_t mblk = ceil_div(M, c.BM), nblk = ceil_div(NS, int64_t(c.WN) * c.SPW);
        const int mode = gemm_kernel_mode();
        if (mode != 2) {
            g.pipe = pipe;
            g.BM = c.BM;
            g.MBLK = int(mblk);
            g.NBLK = int(nblk);
            g.S = 1;
            g.tiles = g.MBLK * g.NBLK;
            return g;
        }
    }
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
    a.KQ = a.KT / a.S;
    a.KR = a.KT % a.S;
    const unsigned blocks = unsigned(round_up(a.tiles, 8));
    void *args[] = {&a};
    const void *fn;
    if (l.shape.pipe >= 0) {
        const PipeCfg &c = kPipeCfg[l.shape.pipe];
        switch (l.shape.pipe) {
        case 0: fn = pipe_kernel_fn<0>(); break;
        case 1: fn = pipe_kernel_fn<1>(); break;
        case 2: fn = pipe_kernel_fn<2>(); break;
        case 3: fn = pipe_kernel_fn<3>(); break;
        case 4: fn = pipe_kernel_fn<4>(); break;
        case 5: fn = pipe_kernel_fn<5>(); break;
        case 6: fn = pipe_kernel_fn<6>(); break;
        case 7: fn = pipe_kernel_fn<7>(); break;
        case 8: fn = pipe_kernel_fn<8>(); break;
        default: fn = pipe_kernel_fn<9>(); break;
        }
        return hipLaunchKernel(fn, dim3(blocks), dim3(unsigned(64 * c.WM * c.WN * c.KS)), args, 0,
                               stream);
    }
    switch (l.shape.BM) {
    case 16: fn = reinterpret_cast<const void *>(&gemm_kernel<16>); break;
    case 32: fn = reinterpret_cast<const void *>(&gemm_kernel<32>); break;
    case 64: fn = reinterpret_cast<const void *>(&gemm_kernel<64>); break;
    default: fn = reinterpret_cast<const void *>(&gemm_kernel<128>); break;
    }
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, stream);
}

}  // namespace w2a8
