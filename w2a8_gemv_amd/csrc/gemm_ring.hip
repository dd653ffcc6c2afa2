// W2A8 batched product for short batches (2 <= M <= 32, K a multiple of 16)
// on gfx950: the GEMV's ring-pipelined weight stream feeding int8 MFMA.
//
// What it computes: the exact integer product of the GEMV
// ("如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？", sections
// "如何判断结果" and "限制与注意事项"; the reference stops at M == 1) for M
// token rows, Y[m][n] = sum_k X[m][k] * W[n][k], plus the fp32 epilogue.
//
// With a few token rows the product is bound by the weight stream, as the
// GEMV is, and its work split is the GEMV ring kernel's: a workgroup owns one
// 32-row strip, or one k-range of it (split strips combine per output with
// the one-atomic word), and splits its tiles over WK waves, each a
// contiguous run.  Each wave keeps a ring of D tiles in flight; a tile
// arrives by direct global->LDS loads (global_load_lds_dwordx4, 1 KiB per
// instruction) into the wave's own ring slot: the packed weight tile, and
// the tile's [8, 16 or 32 rows x 128 k] activations.  The slot is read back
// in MFMA operand order, so no barrier is needed anywhere in the stream.
//
// Per tile a wave issues 2, 3 or 5 load instructions (M up to 8, 16, 32),
// reads 4 weight words and 2 activation fragments per 16-row block per lane
// from LDS, expands the words into signed bytes once, and issues 4
// v_mfma_i32_16x16x64_i8 per 16-row block: A = 16 activation rows x 64 k,
// B = 64 k x 16 weight rows (two 16-row blocks j of the strip, two k-halves
// h of the tile).  Lane l supplies row l % 16 and the 16 bytes of k-group
// l / 16 of each operand.  With M <= 8 the activation rows 8..15 of A repeat
// rows 0..7; their outputs are discarded.
#include "device.h"

namespace w2a8 {
namespace {

#define W2A8_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Wait until at most n vector-memory operations of this wave are
// outstanding (vmcnt only; the compiler does not count global->LDS loads).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait_vm<u * LPT> for u = 0..7 given at run time (a constant once unrolled).
template <int LPT>
__device__ __forceinline__ void wait_vm_tiles(int u) {
    switch (u) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<LPT>(); break;
    case 2: wait_vm<2 * LPT>(); break;
    case 3: wait_vm<3 * LPT>(); break;
    case 4: wait_vm<4 * LPT>(); break;
    case 5: wait_vm<5 * LPT>(); break;
    case 6: wait_vm<6 * LPT>(); break;
    default: wait_vm<7 * LPT>(); break;
    }
}

// Loads of tile t into a ring slot: the weight tile (lane part of the
// permuted slot order) and XL activation parts.
template <int XL>
__device__ __forceinline__ void ring_issue(uint8_t *slot, int t, const int8_t *wsrc,
                                           const int8_t *const *xsrc, int klast) {
    __builtin_amdgcn_global_load_lds(wsrc + int64_t(t) * kTileBytes, W2A8_LDS(slot), 16, 0, 0);
    const int k = min(t * kTileK, klast);
#pragma unroll
    for (int q = 0; q < XL; ++q)
        __builtin_amdgcn_global_load_lds(xsrc[q] + k, W2A8_LDS(slot + kTileBytes * (1 + q)), 16, 0,
                                         0);
}

// The tile in `slot` (its loads have landed): read its operands, then, once
// the reads are done, reissue the slot with tile `refill` (REFILL), then
// the 4*MB MFMAs (each expanded weight word serves the MB row blocks).
template <int XL, int MB, bool REFILL>
__device__ __forceinline__ void ring_consume(uint8_t *slot, int refill, const int (&aoff)[MB][2],
                                             const int (&boff)[2][2], const int8_t *wsrc,
                                             const int8_t *const *xsrc, int klast,
                                             v4i (&acc)[MB][2]) {
    uint32_t bw[2][2];
    v4i av[MB][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int b = 0; b < MB; ++b) av[b][h] = *reinterpret_cast<const v4i *>(slot + aoff[b][h]);
#pragma unroll
        for (int j = 0; j < 2; ++j) bw[j][h] = *reinterpret_cast<const uint32_t *>(slot + boff[j][h]);
    }
    if constexpr (REFILL) {
        // the slot's reads must complete before its loads are reissued
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        ring_issue<XL>(slot, refill, wsrc, xsrc, klast);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const v4i e = expand_word(bw[j][h]);
#pragma unroll
            for (int b = 0; b < MB; ++b)
                acc[b][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[b][h], e, acc[b][j], 0, 0, 0);
        }
}

template <int D, int MR>
__global__ __launch_bounds__(1024) void gemm_ring_kernel(GemvLaunch a) {
    constexpr int XL = MR / 8;                     // activation loads per tile
    constexpr int MB = MR <= 16 ? 1 : MR / 16;     // 16-row blocks of A per tile
    constexpr int LPT = 1 + XL;                    // load instructions per tile
    constexpr int SLOT = kTileBytes * LPT;         // LDS bytes per ring slot
    static_assert(D <= 8, "drain waits cover at most 8 tiles");
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = int(blockIdx.x);
    const int g = int(blockIdx.y);
    const bool big = g < a.KR;
    const int kt0 = g * a.KQ + min(g, a.KR);
    const int ntile = a.KQ + (big ? 1 : 0);
    const int wq = big ? a.WQ1 : a.WQ0, wr = big ? a.WR1 : a.WR0;
    // Tiles of this wave: w0 .. w0+n-1; loads past the run re-read its last
    // tile (an empty run: a tile of this strip).
    const int w0 = kt0 + wv * wq + min(wv, wr);
    const int n = wq + (wv < wr ? 1 : 0);
    const int last = min(max(w0, w0 + n - 1), a.KT - 1);
    uint8_t *ring = smem + wv * (D * SLOT);

    // Weight loads: lane l brings 16-byte slot 8(l>>3) + ((l&7) ^ 2((l>>3)&3))
    // of the tile to LDS position l (an XOR within each group of 8 slots,
    // its own inverse), which makes the B operand reads below hit 32
    // distinct banks.
    const int wslot = 8 * (lane >> 3) + ((lane & 7) ^ (2 * ((lane >> 3) & 3)));
    const int8_t *wsrc = reinterpret_cast<const int8_t *>(a.wp + int64_t(s) * a.KT * kTileWords) +
                         16 * wslot;
    // Activation loads: instruction q, lane l brings row 8q + (l>>3) (rows
    // past M repeat row M-1), 16-byte chunk c = (l&7) ^ (l>>3) of the tile,
    // to position l of part q: chunk c of row r sits at 8(r&7) + (c ^ (r&7)),
    // so that the A fragment reads below spread over the banks.  Chunks past
    // K re-read the row's last chunk; they meet weight padding (code 01,
    // weight 0).
    const int xr = lane >> 3, xc = (lane & 7) ^ (lane >> 3);
    const int8_t *xsrc[XL];
#pragma unroll
    for (int q = 0; q < XL; ++q)
        xsrc[q] = a.x + int64_t(min(8 * q + xr, a.M - 1)) * a.K + 16 * xc;
    const int klast = a.K - 16 - 16 * xc;          // last in-row offset of this lane's chunk

    // Operand offsets within a slot.  B: block j (rows 16j + l%16 of the
    // strip), k-half h (k-group kg = 4h + l/16): word r&3 of lane slot
    // 8(r>>2) + kg, stored at the permuted position.  A, block b: row
    // 16b + l%16, chunk 4h + l/16 (M <= 8: row l%8).
    int boff[2][2], aoff[MB][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 16 * j + (lane & 15);
            const int kg = 4 * h + (lane >> 4);
            const int gq = r >> 2;
            const int pos = 8 * gq + (kg ^ (2 * (gq & 3)));
            boff[j][h] = (pos * 4 + (r & 3)) * 4;
        }
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = MR == 8 ? (lane & 7) : 16 * b + (lane & 15);
            const int c = 4 * h + (lane >> 4);
            aoff[b][h] = kTileBytes * (1 + (r >> 3)) + (8 * (r & 7) + (c ^ (r & 7))) * 16;
        }

    v4i acc[MB][2];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b][0] = acc[b][1] = v4i{0, 0, 0, 0};

    // Fill the ring: tiles w0 .. w0+D-1 (clamped to `last`).
#pragma unroll
    for (int j = 0; j < D; ++j) ring_issue<XL>(ring + j * SLOT, min(w0 + j, last), wsrc, xsrc, klast);

    // Stream: tile i + j of the run sits in slot j; its loads are the oldest
    // D*LPT - (D-1)*LPT outstanding, so waiting down to (D-1)*LPT lands it.
    // The empty asm keeps LDS reads from moving above the wait.
    int i = 0;
    for (; i + D < n; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            wait_vm<(D - 1) * LPT>();
            __asm__ volatile("" ::: "memory");
            ring_consume<XL, MB, true>(ring + j * SLOT, min(w0 + i + D + j, last), aoff, boff, wsrc,
                                   xsrc, klast, acc);
        }
    }
    // The last (at most D) tiles: no refills, so the waits shrink.
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < n) {
            wait_vm_tiles<LPT>(D - 1 - j);
            __asm__ volatile("" ::: "memory");
            ring_consume<XL, MB, false>(ring + j * SLOT, -1, aoff, boff, wsrc, xsrc, klast, acc);
        }
    }
    // Loads issued for a run shorter than the ring may still be writing LDS.
    wait_vm<0>();

    // Outputs.  acc[b][j][e] of lane l is element (m, c) of the strip's
    // [MR x 32] output tile with m = 16b + 4(l/16) + e, c = 16j + l%16.  Each wave
    // writes its tile to the start of its own ring (its loads have all
    // landed, and no other wave touches that ring), so one barrier suffices
    // before the waves read one another's tiles.  The sums are finished in
    // store order: instruction i covers rows 2i (lanes 0..31) and 2i + 1
    // (lanes 32..63), one whole 128-byte row segment each, so no store writes
    // part of a line; with WK waves, wave w finishes the instructions i with
    // i % WK == w.
    {
        int *mine = reinterpret_cast<int *>(ring);
#pragma unroll
        for (int p = 0; p < 8 * MB; ++p) mine[p * 64 + lane] = acc[p >> 3][(p >> 2) & 1][p & 3];
    }
    if (a.WK > 1) __syncthreads();
    constexpr int NI = MR / 2;
    const int c = lane & 31;
    const int Np = a.NS * kTileRows;
    const int row = s * kTileRows + c;
    // the instructions this wave finishes, as a bit mask (no division)
    uint32_t own = 0;
    for (int i = wv; i < NI; i += a.WK) own |= 1u << i;
    const int *red = reinterpret_cast<const int *>(smem);
    constexpr int kRingInts = D * SLOT / 4;        // ints from one wave's ring to the next
    int val[NI], at[NI];
    bool st[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int m = 2 * i + (lane >> 5);
        st[i] = ((own >> i) & 1u) && m < a.M;
        at[i] = ((2 * (m >> 4) + (c >> 4)) * 4 + (m & 3)) * 64 + 16 * ((m >> 2) & 3) + (c & 15);
        val[i] = 0;
    }
    // Sums over the waves' tiles, four waves per step with all their reads in
    // flight (reads past the last wave re-read it and count as zero).
    for (int w = 0; w < a.WK; w += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool ok = w + u < a.WK;
            const int wu = ok ? w + u : a.WK - 1;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int t = red[wu * kRingInts + at[i]];
                val[i] += ok ? t : 0;
            }
        }
    }
    // Every scale load and split-strip atomic is issued before any store, so
    // no wait for a returning value falls between stores (each such wait
    // would also wait for the stores issued before it).
    float sa[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) sa[i] = a.y_f32 && st[i] ? a.sa[2 * i + (lane >> 5)] : 0.0f;
    if (a.SG > 1) {
        uint64_t old[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int m = 2 * i + (lane >> 5);
            if (st[i])
                old[i] = __hip_atomic_fetch_add(a.ws_row + int64_t(m) * Np + row,
                                                split_word(ntile, val[i]), __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int m = 2 * i + (lane >> 5);
            if (st[i])
                st[i] = split_done(a.ws_row + int64_t(m) * Np + row,
                                   old[i] + split_word(ntile, val[i]), a.KT, &val[i]);
        }
    }
    // the scales have landed: one wait here, none between the stores (every
    // value is ready in its own register before the first store: a store's
    // data register is not reused while the store may still read it, which
    // would cost a wait per store)
    if (a.y_f32) wait_vm<0>();
    float fv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) fv[i] = (float(val[i]) * sa[i]) * a.sw;
#pragma unroll
    for (int i = 0; i < NI; ++i) __asm__ volatile("" ::"v"(fv[i]), "v"(val[i]));
    if (row < a.N) {
        if (a.y_i32) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (st[i]) a.y_i32[int64_t(2 * i + (lane >> 5)) * a.N + row] = val[i];
        }
        if (a.y_f32) {
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (st[i]) a.y_f32[int64_t(2 * i + (lane >> 5)) * a.N + row] = fv[i];
        }
    }
}

}  // namespace

size_t gemm_ring_lds_bytes(int M, int wk, int depth) {
    // the waves' slots (at least 4 KiB per wave: they also hold the output
    // exchange of 2 KiB per 16 rows per wave)
    const int mr = M <= 8 ? 8 : M <= 16 ? 16 : 32;
    return size_t(wk) * depth * kTileBytes * (1 + mr / 8);
}

hipError_t launch_gemm_ring(const GemvLaunch &la, int depth, hipStream_t stream) {
    if ((la.K & 15) != 0 || la.M < 1 || la.M > kRingMaxM || la.WK < 1 || la.WK > 16)
        return hipErrorInvalidValue;
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    const int mr = a.M <= 8 ? 8 : a.M <= 16 ? 16 : 32;
    void *args[] = {&a};
    const void *fn;
#define W2A8_GRING(DD)                                                                   \
    fn = mr == 8    ? reinterpret_cast<const void *>(&gemm_ring_kernel<DD, 8>)           \
         : mr == 16 ? reinterpret_cast<const void *>(&gemm_ring_kernel<DD, 16>)          \
                    : reinterpret_cast<const void *>(&gemm_ring_kernel<DD, 32>)
    switch (depth) {
    case 2: W2A8_GRING(2); break;
    case 4: W2A8_GRING(4); break;
    case 6: W2A8_GRING(6); break;
    case 8: W2A8_GRING(8); break;
    default: return hipErrorInvalidValue;
    }
#undef W2A8_GRING
    return hipLaunchKernel(fn, dim3(unsigned(a.NS), unsigned(a.SG)), dim3(unsigned(64 * a.WK)),
                           args, gemm_ring_lds_bytes(a.M, a.WK, depth), stream);
}
#undef W2A8_LDS

}  // namespace w2a8
