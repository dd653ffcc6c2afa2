// W2A8 GEMV (M = 1) for gfx950.
//
// What it computes — "如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？",
// sections "运行 test.py 做 GEMV 基准测试" and "如何判断结果": y equals the
// exact integer product of int8 activations and ternary weights; with the
// scale epilogue of "Windows 上跑通 BitNet b1.58：…部署实录" §3.1
// (the scale is multiplied back after the integer product).
//
// Design (gfx950, wave64):
//  * A workgroup owns one 32-row strip (or, for very long K, one k-range of
//    it) and splits its 1 KiB tiles over WK waves.  Each wave streams a
//    contiguous run of tiles with one 16-byte non-temporal load per lane per
//    tile and keeps up to 2*U tiles in flight; the loads are clamped rather
//    than skipped at the end of the run so the steady state never waits for
//    more than the batch it multiplies.
//  * Each wave stages the activations of its own run into a private LDS
//    region (zero-padded past K, so the ragged last tile needs no special
//    case) and sums them on the way (sum_k x, used below); LDS accesses of one
//    wave are ordered, so this needs no workgroup barrier.  The activation
//    loads are issued before the weight loads, so staging waits only for
//    them.  On small grids (at most 5 waves per CU, K a multiple of 16) the
//    plain kernel skips the staging instead: each lane loads the activation
//    chunk of each tile together with the tile's weights (load_x).
//  * Lane l = 8*rg + kg holds rows 4rg..4rg+3 at k = 16kg..16kg+15 of a tile
//    and reads the matching 16 activation bytes from LDS (a broadcast read).
//  * Decode without sign handling: code c = w + 1 in {0,1,2}.  For a word,
//    the masks 0x03030303, 0x0C0C0C0C, 0x30303030 and (word>>2)&0x30303030
//    leave c, 4c, 16c, 16c in the four bytes, which v_dot4 multiplies with
//    the four activation words; three accumulators (scales 1, 4, 16) are
//    divided back exactly (each partial is a multiple of its scale), and
//    sum_k w*x = sum_k c*x - sum_k x.
//  * Reduction: DPP sums over the 8 lanes of a row group, then the WK waves
//    combine through LDS (one barrier).  Only when a strip's k-range is split
//    over several workgroups do the rows go through the workspace, one
//    device-scope atomic per row and workgroup (split_add in common.h); the
//    last contributor of a row stores it with the epilogue.  Integer addition
//    makes the result independent of arrival order: exact and deterministic.
#include "device.h"

namespace w2a8 {
namespace {

// Activation chunks (16 bytes) staged per lane: a wave's run is at most
// kXChunks * 64 / 8 = 32 tiles (the launch plan keeps RUN <= 32).
constexpr int kXChunks = 4;

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

// Largest |x| of bf16 words (8 values per v4u... 2 per word).
__device__ __forceinline__ float absmax_words(const v4u v, float m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(lo_bf16(v[j])), fabsf(hi_bf16(v[j]))));
    return m;
}

// 16 bf16 activations (two v4u) quantized with `inv`, packed as 16 bytes.
__device__ __forceinline__ v4u quant16(const v4u lo, const v4u hi, float inv) {
    v4u o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t p = w < 2 ? lo[2 * w] : hi[2 * (w - 2)];
        const uint32_t q = w < 2 ? lo[2 * w + 1] : hi[2 * (w - 2) + 1];
        o[w] = q8(lo_bf16(p), inv) | (q8(hi_bf16(p), inv) << 8) | (q8(lo_bf16(q), inv) << 16) |
               (q8(hi_bf16(q), inv) << 24);
    }
    return o;
}

// Bf16 activation chunks that each thread loads, before the weights, for the
// row maximum of the fused kernel (the rest, if any, after them).
constexpr int kAmaxChunks = 2;

// Multiply batch b (only tiles inside the run) against the staged activations.
template <int U>
__device__ __forceinline__ void mac_batch(const v4u (&w)[U], const uint8_t *xl, int w0, int kt0,
                                          int n, int b, int kg, Acc &acc) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (b * U + u < n) {
            const int t = w0 + b * U + u;
            const v4u xv = *reinterpret_cast<const v4u *>(xl + (t - kt0) * kTileK + 16 * kg);
            mac(w[u], xv, acc);
        }
    }
}

// Direct activations: the 16-byte chunk k = 128t + 16kg .. +15 of each tile
// t of batch b, loaded from global memory next to the tile's weights (all
// lanes of a row group read the same 128 bytes, one cache line per tile and
// wave).  Chunks at or past K (K a multiple of 16) load a chunk inside the
// row and are zeroed where they are used, so no load is conditional.
template <int U>
__device__ __forceinline__ void load_x(const int8_t *x, int w0, int last, int b, int kg,
                                       int nchunk, v4u (&xv)[U]) {
    const v4u *xp = reinterpret_cast<const v4u *>(x);
#pragma unroll
    for (int u = 0; u < U; ++u)
        xv[u] = xp[min(min(w0 + b * U + u, last) * (kTileK / 16) + kg, nchunk - 1)];
    __builtin_amdgcn_sched_barrier(0);
}

// Multiply batch b against its directly loaded activation chunks, and add
// those chunks' sum to sxl.
template <int U>
__device__ __forceinline__ void mac_batch_dx(const v4u (&w)[U], const v4u (&xv)[U], int w0,
                                             int n, int b, int kg, int K, Acc &acc, int &sxl) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (b * U + u < n) {
            const int t = w0 + b * U + u;
            const bool in = t * kTileK + 16 * kg < K;
            const v4u x = in ? xv[u] : v4u{0u, 0u, 0u, 0u};
            mac(w[u], x, acc);
            sxl = dot4(x[0], 0x01010101u, sxl);
            sxl = dot4(x[1], 0x01010101u, sxl);
            sxl = dot4(x[2], 0x01010101u, sxl);
            sxl = dot4(x[3], 0x01010101u, sxl);
        }
    }
}

// FUSED: the activations arrive as one bf16 row (a.xb).  Every workgroup
// takes the row's largest |x| itself, quantizes its own k-range with the same
// per-element operations as the quantizer kernel (q8 in common.h) and scale
// s_a = amax/127, so the result is bit-identical to quant_act_int8 followed
// by the plain GEMV, in one launch.
// GROUPED: the strip's matrix, outputs and weight scale come from the
// projection table t (select_proj); the split-k workspace words are indexed
// by the strip's position in the whole launch.
// DX (not FUSED, K a multiple of 16): activation chunks are loaded with each
// batch of weights straight into registers (load_x) instead of being staged
// through LDS first, which removes the staging and its wait from the start
// of every wave.
template <int U, bool FUSED, bool GROUPED, bool DX>
__device__ __forceinline__ void gemv_body(const GemvLaunch a, const GemvGroups t) {
    static_assert(!(FUSED && DX), "the fused kernel quantizes its staged chunks");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Strip s, k-range g of it, and this wave's run of tiles, from quotients
    // and remainders the launcher computed: a division here (64-bit, in
    // software) would cost hundreds of scalar instructions before the first
    // load.
    const int s = int(blockIdx.x);
    const int g = int(blockIdx.y);
    const Proj pj = select_proj<GROUPED>(a, t, s);
    const bool big = g < a.KR;
    const int kt0 = g * a.KQ + min(g, a.KR);
    const int ntile = a.KQ + (big ? 1 : 0);
    const int wq = big ? a.WQ1 : a.WQ0, wr = big ? a.WR1 : a.WR0;
    const int w0 = kt0 + wv * wq + min(wv, wr);
    const int n = wq + (wv < wr ? 1 : 0);
    const int w1 = w0 + n;
    const int nb = (n + U - 1) / U;
    const int kg = lane & 7, rg = lane >> 3;

    // LDS: per-wave activation regions of RUN tiles (not with DX), then the
    // row partials.
    uint8_t *xl = smem + wv * (a.RUN * kTileK);
    int *red = reinterpret_cast<int *>(smem + (DX ? 0 : a.WK * a.RUN * kTileK));   // WK*32 ints

    const v4u *wt =
        reinterpret_cast<const v4u *>(pj.wp + int64_t(pj.s) * a.KT * kTileWords) + lane;
    // Last tile a load may touch: the run's last tile, or (for an empty run)
    // a tile of this strip, never past it.
    const int last = min(max(w0, w1 - 1), a.KT - 1);

    // 1. This wave's activation chunks (k in [w0*128, w1*128)) that lie
    //    entirely below K, at most kXChunks per lane, loaded before the
    //    weights so that staging waits only for them.  The one chunk that
    //    straddles K (only when K % 16 != 0) is assembled byte by byte.
    const int kbase = w0 * kTileK;
    const int nchunk = n * (kTileK / 16);
    v4u xr[kXChunks];
    // Fused: the run's 16-value chunks as bf16 (two v4u each) and this
    // thread's share of the whole row for its maximum.
    v4u xh[FUSED ? kXChunks : 1][2];
    v4u am[FUSED ? kAmaxChunks : 1][2];
    const int nfull = a.K >> 4;                    // 16-value chunks entirely below K
    const int nthr = 64 * a.WK;
    if constexpr (FUSED) {
#pragma unroll
        for (int j = 0; j < kXChunks; ++j) {
            const int c = lane + 64 * j;
            xh[j][0] = xh[j][1] = v4u{0u, 0u, 0u, 0u};
            if (c < nchunk && kbase + 16 * c + 16 <= a.K) {
                const v4u *p = reinterpret_cast<const v4u *>(a.xb + kbase + 16 * c);
                xh[j][0] = p[0];
                xh[j][1] = p[1];
            }
        }
#pragma unroll
        for (int i = 0; i < kAmaxChunks; ++i) {
            const int c = tid + nthr * i;
            am[i][0] = am[i][1] = v4u{0u, 0u, 0u, 0u};
            if (c < nfull) {
                const v4u *p = reinterpret_cast<const v4u *>(a.xb + 16 * c);
                am[i][0] = p[0];
                am[i][1] = p[1];
            }
        }
    } else if constexpr (!DX) {
#pragma unroll
        for (int j = 0; j < kXChunks; ++j) {
            const int c = lane + 64 * j;
            xr[j] = v4u{0u, 0u, 0u, 0u};
            if (c < nchunk && kbase + 16 * c + 16 <= a.K)
                xr[j] = *reinterpret_cast<const v4u *>(a.x + kbase + 16 * c);
        }
    }
    if (!FUSED && !DX && (a.K & 15) != 0) {
#pragma unroll
        for (int j = 0; j < kXChunks; ++j) {
            const int c = lane + 64 * j;
            const int k0 = kbase + 16 * c;
            if (c < nchunk && k0 < a.K && k0 + 16 > a.K) {
                uint32_t b4[4] = {0u, 0u, 0u, 0u};
                for (int i = 0; i < 16; ++i)
                    if (k0 + i < a.K)
                        b4[i >> 2] |= uint32_t(uint8_t(a.x[k0 + i])) << (8 * (i & 3));
                xr[j] = v4u{b4[0], b4[1], b4[2], b4[3]};
            }
        }
    }

    // 2. Two batches of weight loads in flight (clamped to the run, so the
    //    count of outstanding loads is the same in every wave).
    v4u wa[U], wb[U];
    v4u xva[DX ? U : 1], xvb[DX ? U : 1];
    const int xchunks = a.K >> 4;
    load_batch<U>(wt, w0, last, 0, wa);
    if constexpr (DX) load_x<U>(a.x, w0, last, 0, kg, xchunks, xva);
    load_batch<U>(wt, w0, last, 1, wb);
    if constexpr (DX) load_x<U>(a.x, w0, last, 1, kg, xchunks, xvb);

    // 2b. Fused: the row maximum (chunks beyond the first share and the
    //     values past the last whole chunk after the weight loads), combined
    //     over the workgroup through LDS; then this run's codes.
    float sa = 0.0f;
    if constexpr (FUSED) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kAmaxChunks; ++i)
            amax = absmax_words(am[i][1], absmax_words(am[i][0], amax));
        for (int c = tid + nthr * kAmaxChunks; c < nfull; c += nthr) {
            const v4u *p = reinterpret_cast<const v4u *>(a.xb + 16 * c);
            amax = absmax_words(p[1], absmax_words(p[0], amax));
        }
        if (tid == 0)
            for (int k = 16 * nfull; k < a.K; ++k)
                amax = fmaxf(amax, fabsf(__uint_as_float(uint32_t(a.xb[k]) << 16)));
        amax = wave_max_nonneg(amax);
        // across the waves: each writes its maximum, the unused entries of
        // the 16 are zeroed, and every lane reads all 16 with four 16-byte
        // reads
        float *fred = reinterpret_cast<float *>(red + a.WK * kTileRows);   // 16 floats
        if (lane == 0) fred[wv] = amax;
        if (tid >= a.WK && tid < 16) fred[tid] = 0.0f;
        __syncthreads();
        {
            const v4u *r4 = reinterpret_cast<const v4u *>(fred);
            const v4u q0 = r4[0], q1 = r4[1], q2 = r4[2], q3 = r4[3];
            float m4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m4[i] = fmaxf(fmaxf(__uint_as_float(q0[i]), __uint_as_float(q1[i])),
                              fmaxf(__uint_as_float(q2[i]), __uint_as_float(q3[i])));
            amax = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        }
        // The quantizer's scale and reciprocal; a zero row quantizes to 0.
        sa = amax / 127.0f;
        const float inv = amax == 0.0f ? 0.0f : fminf(127.0f / amax, __FLT_MAX__);
#pragma unroll
        for (int j = 0; j < kXChunks; ++j) {
            const int c = lane + 64 * j;
            xr[j] = v4u{0u, 0u, 0u, 0u};
            if (64 * j >= nchunk) continue;   // the whole group lies past the run
            xr[j] = quant16(xh[j][0], xh[j][1], inv);
            const int k0 = kbase + 16 * c;
            if ((a.K & 15) != 0 && c < nchunk && k0 < a.K && k0 + 16 > a.K) {
                uint32_t b4[4] = {0u, 0u, 0u, 0u};
                for (int i = 0; i < 16; ++i)
                    if (k0 + i < a.K)
                        b4[i >> 2] |= q8(__uint_as_float(uint32_t(a.xb[k0 + i]) << 16), inv)
                                      << (8 * (i & 3));
                xr[j] = v4u{b4[0], b4[1], b4[2], b4[3]};
            }
        }
    }

    // 3. Stage the run's activations into the wave's LDS region and sum them.
    int sx = 0;
    if constexpr (!DX) {
#pragma unroll
        for (int j = 0; j < kXChunks; ++j) {
            const int c = lane + 64 * j;
            if (c < nchunk) *reinterpret_cast<v4u *>(xl + 16 * c) = xr[j];
            sx = dot4(xr[j][0], 0x01010101u, sx);
            sx = dot4(xr[j][1], 0x01010101u, sx);
            sx = dot4(xr[j][2], 0x01010101u, sx);
            sx = dot4(xr[j][3], 0x01010101u, sx);
        }
        sx = wave_sum(sx);
    }

    // 4. Stream the run: multiply one batch while the next is in flight.
    Acc acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
    if constexpr (DX) {
        // Each lane sums its own chunks (kg) of the run; the 8 lanes of a
        // row group together hold every chunk once.
        int sxl = 0;
        if (n > 0) {
            int b = 0;
            for (; b + 2 < nb; b += 2) {
                mac_batch_dx<U>(wa, xva, w0, n, b, kg, a.K, acc, sxl);
                load_batch<U>(wt, w0, last, b + 2, wa);
                load_x<U>(a.x, w0, last, b + 2, kg, xchunks, xva);
                mac_batch_dx<U>(wb, xvb, w0, n, b + 1, kg, a.K, acc, sxl);
                load_batch<U>(wt, w0, last, b + 3, wb);
                load_x<U>(a.x, w0, last, b + 3, kg, xchunks, xvb);
            }
            mac_batch_dx<U>(wa, xva, w0, n, b, kg, a.K, acc, sxl);
            if (b + 1 < nb) mac_batch_dx<U>(wb, xvb, w0, n, b + 1, kg, a.K, acc, sxl);
        }
        sx = sum8(sxl);
    } else if (n > 0) {
        int b = 0;
        for (; b + 2 < nb; b += 2) {
            mac_batch<U>(wa, xl, w0, w0, n, b, kg, acc);
            load_batch<U>(wt, w0, last, b + 2, wa);
            mac_batch<U>(wb, xl, w0, w0, n, b + 1, kg, acc);
            load_batch<U>(wt, w0, last, b + 3, wb);
        }
        mac_batch<U>(wa, xl, w0, w0, n, b, kg, acc);
        if (b + 1 < nb) mac_batch<U>(wb, xl, w0, w0, n, b + 1, kg, acc);
    }

    // 5. Reduce: 8 lanes per row group (DPP); sum_k w*x = sum_k c*x - sum_k x
    //    over the wave's run; then the WK waves via LDS.
    int r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = sum8(acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4));
    // Lane (rg, kg) with kg < 4 owns row 4rg + kg of the strip.
    const int mine = (kg == 0 ? r[0] : kg == 1 ? r[1] : kg == 2 ? r[2] : r[3]) - sx;
    int tot = 0;
    int r32;   // row within the strip
    bool owner;
    if (a.WK == 1) {
        tot = mine;
        r32 = rg * 4 + kg;
        owner = kg < 4;
    } else {
        if (kg < 4) red[wv * kTileRows + rg * 4 + kg] = mine;
        __syncthreads();
        r32 = tid;
        owner = tid < kTileRows;
        if (owner)
            for (int w = 0; w < a.WK; ++w) tot += red[w * kTileRows + tid];
    }
    const int row = pj.s * kTileRows + r32;

    if constexpr (!FUSED) sa = pj.y_f32 ? a.sa[0] : 0.0f;
    if (a.SG == 1) {
        if (owner && row < pj.N) store_proj(pj, sa, row, tot);
        return;
    }
    // k-range split over workgroups: one device-scope atomic per row (coherent
    // across the XCDs' L2s) combines the partials; the last contributor of a
    // row stores it.
    int v;
    if (owner && split_add(a.ws_row + s * kTileRows + r32, ntile, tot, a.KT, &v) && row < pj.N)
        store_proj(pj, sa, row, v);
}

template <int U, bool FUSED, bool DX = false>
__global__ __launch_bounds__(1024) void gemv_kernel(GemvLaunch a) {
    gemv_body<U, FUSED, false, DX>(a, GemvGroups{});
}

template <int U, bool FUSED, bool DX = false>
__global__ __launch_bounds__(1024) void gemv_grouped_kernel(GemvLaunch a, GemvGroups t) {
    gemv_body<U, FUSED, true, DX>(a, t);
}


// ---------------------------------------------------------------------------
// Few activation rows (2 <= M <= MR <= 8): the product of a short batch of
// tokens with the same weight stream.  Same work split, layout, loads and
// reductions as gemv_kernel; each lane decodes its weight words once (codes
// c = w + 1 as bytes) and multiplies them against the M activation rows, each row
// staged in its own LDS region of the wave (runs of at most 8 tiles, one
// 16-byte chunk per lane per row).  Rows are y[m][n], row-major.
// ---------------------------------------------------------------------------
// With several rows the codes are shifted back to bytes 0..2 once per word
// (shared by the rows), so each row keeps one accumulator per word instead
// of three scaled ones: registers, not VALU, limit this kernel.
struct AccR {
    int a[4];
};

template <int MR>
__device__ __forceinline__ void mac_rows(const v4u w, const v4u (&xv)[MR], AccR (&acc)[MR]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        const uint32_t c0 = v & 0x03030303u, c1 = (v >> 2) & 0x03030303u,
                       c2 = (v >> 4) & 0x03030303u, c3 = (v >> 6) & 0x03030303u;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            int s = dot4(c0, xv[m][0], acc[m].a[q]);
            s = dot4(c1, xv[m][1], s);
            s = dot4(c2, xv[m][2], s);
            acc[m].a[q] = dot4(c3, xv[m][3], s);
        }
    }
}

template <int U, int MR>
__device__ __forceinline__ void mac_batch_rows(const v4u (&w)[U], const uint8_t *xl, int rstride,
                                               int n, int b, int kg, AccR (&acc)[MR]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (b * U + u < n) {
            v4u xv[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m)
                xv[m] = *reinterpret_cast<const v4u *>(xl + m * rstride + (b * U + u) * kTileK +
                                                       16 * kg);
            mac_rows<MR>(w[u], xv, acc);
        }
    }
}

// At most 32/MR waves per workgroup (the plan's limit), which leaves room
// for MR rows of accumulators without spilling.
template <int U, int MR>
__global__ __launch_bounds__(2048 / MR) __attribute__((amdgpu_waves_per_eu(3)))
void gemv_rows_kernel(GemvLaunch a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = int(blockIdx.x);
    const int g = int(blockIdx.y);
    const bool big = g < a.KR;
    const int kt0 = g * a.KQ + min(g, a.KR);
    const int ntile = a.KQ + (big ? 1 : 0);
    const int wq = big ? a.WQ1 : a.WQ0, wr = big ? a.WR1 : a.WR0;
    const int w0 = kt0 + wv * wq + min(wv, wr);
    const int n = wq + (wv < wr ? 1 : 0);
    const int w1 = w0 + n;
    const int nb = (n + U - 1) / U;
    const int kg = lane & 7, rg = lane >> 3;
    const int M = a.M;

    // LDS: per wave MR row regions of RUN tiles, then WK*MR*32 row partials.
    const int rstride = a.RUN * kTileK;
    uint8_t *xl = smem + wv * (MR * rstride);
    int *red = reinterpret_cast<int *>(smem + a.WK * MR * rstride);

    const v4u *wt = reinterpret_cast<const v4u *>(a.wp + int64_t(s) * a.KT * kTileWords) + lane;
    const int last = min(max(w0, w1 - 1), a.KT - 1);

    // 1. Activation chunk `lane` of the run for each row (runs are at most 8
    //    tiles: 64 chunks), before the weights; rows past M are zero.
    const int kbase = w0 * kTileK;
    const int nchunk = n * (kTileK / 16);
    const int k0 = kbase + 16 * lane;
    // Rows are 16-byte aligned only when K % 16 == 0; otherwise every chunk
    // is assembled byte by byte (and the one straddling K is zero-padded).
    v4u xr[MR];
    const bool xvec = (a.K & 15) == 0;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        xr[m] = v4u{0u, 0u, 0u, 0u};
        if (xvec && m < M && lane < nchunk && k0 + 16 <= a.K)
            xr[m] = *reinterpret_cast<const v4u *>(a.x + int64_t(m) * a.K + k0);
    }
    if (!xvec && lane < nchunk && k0 < a.K) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= M) continue;
            uint32_t b4[4] = {0u, 0u, 0u, 0u};
            for (int i = 0; i < 16; ++i)
                if (k0 + i < a.K)
                    b4[i >> 2] |= uint32_t(uint8_t(a.x[int64_t(m) * a.K + k0 + i])) << (8 * (i & 3));
            xr[m] = v4u{b4[0], b4[1], b4[2], b4[3]};
        }
    }

    // 2. Two batches of weight loads in flight.
    v4u wa[U], wb[U];
    load_batch<U>(wt, w0, last, 0, wa);
    load_batch<U>(wt, w0, last, 1, wb);

    // 3. Stage each row's chunk in its LDS region and sum the rows.
    int sx[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (lane < nchunk) *reinterpret_cast<v4u *>(xl + m * rstride + 16 * lane) = xr[m];
        int t = dot4(xr[m][0], 0x01010101u, 0);
        t = dot4(xr[m][1], 0x01010101u, t);
        t = dot4(xr[m][2], 0x01010101u, t);
        t = dot4(xr[m][3], 0x01010101u, t);
        sx[m] = wave_sum(t);
    }

    // 4. Stream the run.
    AccR acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[m].a[q] = 0;
    if (n > 0) {
        int b = 0;
        for (; b + 2 < nb; b += 2) {
            mac_batch_rows<U, MR>(wa, xl, rstride, n, b, kg, acc);
            load_batch<U>(wt, w0, last, b + 2, wa);
            mac_batch_rows<U, MR>(wb, xl, rstride, n, b + 1, kg, acc);
            load_batch<U>(wt, w0, last, b + 3, wb);
        }
        mac_batch_rows<U, MR>(wa, xl, rstride, n, b, kg, acc);
        if (b + 1 < nb) mac_batch_rows<U, MR>(wb, xl, rstride, n, b + 1, kg, acc);
    }

    // 5. Per row: 8 lanes per row group, the run's sum x, then the waves.
    int tot[MR];
    int row;
    bool owner;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        int r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = sum8(acc[m].a[q]);
        tot[m] = (kg == 0 ? r[0] : kg == 1 ? r[1] : kg == 2 ? r[2] : r[3]) - sx[m];
    }
    if (a.WK == 1) {
        row = s * kTileRows + rg * 4 + kg;
        owner = kg < 4;
    } else {
        if (kg < 4)
#pragma unroll
            for (int m = 0; m < MR; ++m) red[(m * a.WK + wv) * kTileRows + rg * 4 + kg] = tot[m];
        __syncthreads();
        row = s * kTileRows + tid;
        owner = tid < kTileRows;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            tot[m] = 0;
            if (owner)
                for (int w = 0; w < a.WK; ++w) tot[m] += red[(m * a.WK + w) * kTileRows + tid];
        }
    }
    if (!owner) return;
    const int64_t Np = int64_t(a.NS) * kTileRows;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m >= M) break;
        int v = tot[m];
        if (a.SG > 1 && !split_add(a.ws_row + m * Np + row, ntile, tot[m], a.KT, &v)) continue;
        if (row < a.N) {
            const int64_t o = int64_t(m) * a.N + row;
            if (a.y_i32) a.y_i32[o] = v;
            if (a.y_f32) a.y_f32[o] = (float(v) * a.sa[m]) * a.sw;
        }
    }
}

}  // namespace

size_t gemv_rows_lds_bytes(const GemvLaunch &a, int MR) {
    return size_t(a.WK) * MR * a.RUN * kTileK + size_t(a.WK) * MR * kTileRows * 4;
}

hipError_t launch_gemv_rows(const GemvLaunch &la, hipStream_t stream) {
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    void *args[] = {&a};
    const int MR = a.M <= 2 ? 2 : a.M <= 4 ? 4 : 8;
    const void *fn;
    switch (MR * 10 + a.unroll) {
    case 22: fn = reinterpret_cast<const void *>(&gemv_rows_kernel<2, 2>); break;
    case 24: fn = reinterpret_cast<const void *>(&gemv_rows_kernel<4, 2>); break;
    case 42: fn = reinterpret_cast<const void *>(&gemv_rows_kernel<2, 4>); break;
    case 44: fn = reinterpret_cast<const void *>(&gemv_rows_kernel<4, 4>); break;
    case 82: fn = reinterpret_cast<const void *>(&gemv_rows_kernel<2, 8>); break;
    default: fn = reinterpret_cast<const void *>(&gemv_rows_kernel<4, 8>); break;
    }
    return hipLaunchKernel(fn, dim3(unsigned(a.NS), unsigned(a.SG)), dim3(unsigned(64 * a.WK)),
                           args, gemv_rows_lds_bytes(a, MR), stream);
}

size_t gemv_lds_bytes(const GemvLaunch &a) {
    // activation regions, row partials, and the fused kernel's per-wave maxima
    return size_t(a.WK) * a.RUN * kTileK + size_t(a.WK) * kTileRows * 4 + 16 * 4;
}

// Direct activation loads (no LDS staging) for the plain kernel when the grid
// has at most 5 waves per CU, K is a multiple of 16 and the load batch is at
// most 4 tiles.  Measured on MI355X (cold, interleaved runs): 0.02-0.07 us
// less on each of the six sweep shapes of 640 to 1200 waves, but 0.09 us more
// at 13824 x 2560 (1728 waves), 0.33 us more at 20480 x 3200 (2560) and
// 1.15 us more at 5120 x 27648 (5760), where the extra 64-lane load
// instruction per tile costs more than the staging it saves.
// The chunks also take 2U more registers per lane, which a batch of 8 would
// push past the budget of 16-wave workgroups.
static bool gemv_direct_x(const GemvLaunch &a) {
    return a.DXOK && a.xb == nullptr && (a.K & 15) == 0 && a.unroll <= 4;
}

static size_t gemv_launch_lds_bytes(const GemvLaunch &a) {
    return gemv_direct_x(a) ? size_t(a.WK) * kTileRows * 4 : gemv_lds_bytes(a);
}

hipError_t launch_gemv(const GemvLaunch &la, hipStream_t stream) {
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    void *args[] = {&a};
    const void *fn;
    const bool fused = a.xb != nullptr;
    const bool dx = gemv_direct_x(a);
    switch (a.unroll * 2 + (fused ? 1 : 0)) {
    case 4:
        fn = dx ? reinterpret_cast<const void *>(&gemv_kernel<2, false, true>)
                : reinterpret_cast<const void *>(&gemv_kernel<2, false>);
        break;
    case 5: fn = reinterpret_cast<const void *>(&gemv_kernel<2, true>); break;
    case 8:
        fn = dx ? reinterpret_cast<const void *>(&gemv_kernel<4, false, true>)
                : reinterpret_cast<const void *>(&gemv_kernel<4, false>);
        break;
    case 9: fn = reinterpret_cast<const void *>(&gemv_kernel<4, true>); break;
    case 17: fn = reinterpret_cast<const void *>(&gemv_kernel<8, true>); break;
    default: fn = reinterpret_cast<const void *>(&gemv_kernel<8, false>); break;
    }
    // x: strip, y: k-range of the strip.
    return hipLaunchKernel(fn, dim3(unsigned(a.NS), unsigned(a.SG)), dim3(unsigned(64 * a.WK)),
                           args, gemv_launch_lds_bytes(a), stream);
}

hipError_t launch_gemv_fused(const GemvLaunch &a, hipStream_t stream) {
    return a.xb ? launch_gemv(a, stream) : hipErrorInvalidValue;
}

hipError_t launch_gemv_grouped(const GemvLaunch &la, const GemvGroups &t, hipStream_t stream) {
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    GemvGroups tt = t;
    void *args[] = {&a, &tt};
    const void *fn;
    const bool fused = a.xb != nullptr;
    const bool dx = gemv_direct_x(a);
    switch (a.unroll * 2 + (fused ? 1 : 0)) {
    case 4:
        fn = dx ? reinterpret_cast<const void *>(&gemv_grouped_kernel<2, false, true>)
                : reinterpret_cast<const void *>(&gemv_grouped_kernel<2, false>);
        break;
    case 5: fn = reinterpret_cast<const void *>(&gemv_grouped_kernel<2, true>); break;
    case 8:
        fn = dx ? reinterpret_cast<const void *>(&gemv_grouped_kernel<4, false, true>)
                : reinterpret_cast<const void *>(&gemv_grouped_kernel<4, false>);
        break;
    case 9: fn = reinterpret_cast<const void *>(&gemv_grouped_kernel<4, true>); break;
    case 17: fn = reinterpret_cast<const void *>(&gemv_grouped_kernel<8, true>); break;
    default: fn = reinterpret_cast<const void *>(&gemv_grouped_kernel<8, false>); break;
    }
    return hipLaunchKernel(fn, dim3(unsigned(a.NS), unsigned(a.SG)), dim3(unsigned(64 * a.WK)),
                           args, gemv_launch_lds_bytes(a), stream);
}

}  // namespace w2a8
