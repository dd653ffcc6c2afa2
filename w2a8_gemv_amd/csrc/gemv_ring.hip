// W2A8 GEMV (M = 1) for gfx950: ring-pipelined weight stream.
//
// What it computes — "如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？",
// sections "运行 test.py 做 GEMV 基准测试" and "如何判断结果": y equals the
// exact integer product of int8 activations and ternary weights; with the
// scale epilogue of "Windows 上跑通 BitNet b1.58：…部署实录" §3.1.
//
// Same work split, layout, decode and reductions as the batch kernel
// (gemv.hip): a workgroup owns one 32-row strip, or one k-range of it, and
// splits its tiles over WK waves, each a contiguous run.  What differs is the
// weight stream: each wave keeps a ring of D tiles in flight and consumes one
// tile at a time, reloading its slot with the tile D further on, so D-1 loads
// stay outstanding throughout the run (loads return in order, so the wait
// before each tile is exact).  Plain reads of this device reach their best
// rate with about four waves per CU and 8 to 12 KiB in flight per wave; a
// ring holds that depth over a long run with one wave per SIMD, where the
// batch kernel's two batches of U tiles halve the depth between refills.
//
// Tile addresses are wave-uniform (scalar base + lane offset), so the ring
// costs no vector instructions besides the multiply.  Activations (K a
// multiple of 16): each lane loads its tile's 16-byte chunk next to the
// weights (a second ring, L2 hits), and Σx is summed from the same chunks.
#include "device.h"

namespace w2a8 {
namespace {

struct RingAcc {
    int a1[4], a4[4], a16[4];
};

// One lane slot of a tile: 4 rows x 16 k of codes c = w + 1 against 16
// activation bytes.  Masks leave c, 4c, 16c, 16c in the bytes; three
// accumulators (scales 1, 4, 16) are divided back exactly at the end.
__device__ __forceinline__ void ring_mac(const v4u w, const v4u xv, RingAcc &acc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        acc.a1[q] = dot4(v & 0x03030303u, xv[0], acc.a1[q]);
        acc.a4[q] = dot4(v & 0x0C0C0C0Cu, xv[1], acc.a4[q]);
        acc.a16[q] = dot4(v & 0x30303030u, xv[2], acc.a16[q]);
        acc.a16[q] = dot4((v >> 2) & 0x30303030u, xv[3], acc.a16[q]);
    }
}

__device__ __forceinline__ int xsum16(const v4u x, int s) {
    s = dot4(x[0], 0x01010101u, s);
    s = dot4(x[1], 0x01010101u, s);
    s = dot4(x[2], 0x01010101u, s);
    return dot4(x[3], 0x01010101u, s);
}

// GROUPED: the strip's matrix, outputs and weight scale come from the
// projection table (strips numbered across the projections); the split-k
// combining words are indexed by the strip's position in the whole launch.
template <int D, bool GROUPED>
__device__ __forceinline__ void ring_body(const GemvLaunch &a, const GemvGroups &tab) {
    __shared__ int red[16 * kTileRows];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = int(blockIdx.x);
    const int g = int(blockIdx.y);
    const Proj pj = select_proj<GROUPED>(a, tab, s);
    const bool big = g < a.KR;
    const int kt0 = g * a.KQ + min(g, a.KR);
    const int ntile = a.KQ + (big ? 1 : 0);
    const int wq = big ? a.WQ1 : a.WQ0, wr = big ? a.WR1 : a.WR0;
    // Tiles of this wave: w0 .. w0+n-1.
    const int w0 = kt0 + wv * wq + min(wv, wr);
    const int n = wq + (wv < wr ? 1 : 0);
    const int kg = lane & 7, rg = lane >> 3;
    // Last tile a load may touch: the run's last tile (or, for an empty run,
    // a tile of this strip).
    const int last = min(max(w0, w0 + n - 1), a.KT - 1);
    const v4u *sbase = reinterpret_cast<const v4u *>(pj.wp + int64_t(pj.s) * a.KT * kTileWords);

    // 1. Fill the ring: tiles w0 .. w0+D-1 (clamped to `last`) and their
    //    activation chunks.
    v4u r[D], xq[D];
    const v4u *xp = reinterpret_cast<const v4u *>(a.x);
    const int xlast = (a.K >> 4) - 1;          // last 16-byte chunk (K % 16 == 0)
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(w0 + j, last);
        r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + lane);
        xq[j] = xp[min(t * (kTileK / 16) + kg, xlast)];
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. Stream: consume tile i of the run, reload its slot with tile i + D.
    RingAcc acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
    int sxl = 0;
    int i = 0;
    for (; i + D < n; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            sxl = xsum16(xq[j], sxl);
            ring_mac(r[j], xq[j], acc);
            const int t = min(w0 + i + D + j, last);
            r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + lane);
            xq[j] = xp[min(t * (kTileK / 16) + kg, xlast)];
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < n) {
            // chunks at or past K count as zero: only the strip's last tile
            // can reach past K, and it is always among the run's last D
            const bool in = (w0 + i + j) * kTileK + 16 * kg < a.K;
            const v4u xv = in ? xq[j] : v4u{0u, 0u, 0u, 0u};
            sxl = xsum16(xv, sxl);
            ring_mac(r[j], xv, acc);
        }
    }
    const int sx = sum8(sxl);

    // 3. Reduce: 8 lanes per row group; sum_k w*x = sum_k c*x - sum_k x over
    //    the run; then the WK waves via LDS.
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rr[q] = sum8(acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4));
    const int mine = (kg == 0 ? rr[0] : kg == 1 ? rr[1] : kg == 2 ? rr[2] : rr[3]) - sx;
    int tot = 0, r32;
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
    const float sa = pj.y_f32 ? a.sa[0] : 0.0f;
    int v = tot;
    if (a.SG > 1 &&
        !(owner && split_add(a.ws_row + s * kTileRows + r32, ntile, tot, a.KT, &v)))
        return;
    if (owner && row < pj.N) store_proj(pj, sa, row, v);
}

template <int D>
__global__ __launch_bounds__(1024) void gemv_ring_kernel(GemvLaunch a) {
    ring_body<D, false>(a, GemvGroups{});
}

template <int D>
__global__ __launch_bounds__(1024) void gemv_ring_grouped_kernel(GemvLaunch a, GemvGroups t) {
    ring_body<D, true>(a, t);
}

// Row-slice variant for matrices with few strips: kSlices single-wave
// workgroups share a strip, workgroup (s, sl) owning the 4 rows of row group
// sl in every tile of strip s.  A step reads the 128-byte slice of 8
// consecutive tiles (lane l: tile l/8 of the step, k-chunk l%8), so a strip
// is read by 8 waves spread over the device without splitting its k-range:
// no combining words and no atomics.  Each lane holds 4 rows x 16 k of one
// tile; a row's value is the sum over the whole wave.  GROUPED: strips are
// numbered across the projections, as in the grouped ring kernel.
constexpr int kSlices = 8;

template <int D, bool GROUPED>
__device__ __forceinline__ void slice_body(const GemvLaunch &a, const GemvGroups &tab) {
    const int lane = threadIdx.x;
    const int s = int(blockIdx.x) / kSlices, sl = int(blockIdx.x) % kSlices;
    const Proj pj = select_proj<GROUPED>(a, tab, s);
    const int u = lane >> 3, kg = lane & 7;     // tile of the step, k-chunk
    const int off = sl * 8 + kg;                // 16-byte slot within a tile
    const int nst = (a.KT + kSlices - 1) / kSlices;
    const int last = a.KT - 1;
    const v4u *sbase = reinterpret_cast<const v4u *>(pj.wp + int64_t(pj.s) * a.KT * kTileWords);
    const v4u *xp = reinterpret_cast<const v4u *>(a.x);
    const int xlast = (a.K >> 4) - 1;           // last 16-byte chunk (K % 16 == 0)

    // 1. Fill the ring: steps 0 .. D-1 (tiles clamped to the strip's last).
    v4u r[D], xq[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(j * kSlices + u, last);
        r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + off);
        xq[j] = xp[min(t * (kTileK / 16) + kg, xlast)];
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. Stream: every step but the last is whole and inside K (the strip's
    //    last tile is in the last step).
    RingAcc acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
    int sxl = 0;
    int i = 0;
    for (; i + D < nst; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            sxl = xsum16(xq[j], sxl);
            ring_mac(r[j], xq[j], acc);
            const int t = min((i + D + j) * kSlices + u, last);
            r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + off);
            xq[j] = xp[min(t * (kTileK / 16) + kg, xlast)];
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < nst) {
            // lanes past the strip's last tile, and chunks at or past K, count as zero
            const int t = (i + j) * kSlices + u;
            const bool in = t <= last && t * kTileK + 16 * kg < a.K;
            const v4u xv = in ? xq[j] : v4u{0u, 0u, 0u, 0u};
            sxl = xsum16(xv, sxl);
            ring_mac(r[j], xv, acc);
        }
    }

    // 3. Reduce over the wave: sum_k w*x = sum_k c*x - sum_k x per row.
    const int sx = wave_sum(sxl);
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rr[q] = wave_sum(acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4));
    if (lane >= 4) return;
    const int v = (lane == 0 ? rr[0] : lane == 1 ? rr[1] : lane == 2 ? rr[2] : rr[3]) - sx;
    const int row = pj.s * kTileRows + sl * 4 + lane;
    const float sa = pj.y_f32 ? a.sa[0] : 0.0f;
    if (row < pj.N) store_proj(pj, sa, row, v);
}

template <int D>
__global__ __launch_bounds__(64) void gemv_slice_kernel(GemvLaunch a) {
    slice_body<D, false>(a, GemvGroups{});
}

template <int D>
__global__ __launch_bounds__(64) void gemv_slice_grouped_kernel(GemvLaunch a, GemvGroups t) {
    slice_body<D, true>(a, t);
}

}  // namespace

// Ring-kernel plan (K a multiple of 16): plain reads of this device reach
// their best rate with ~10-12 MB in flight spread over all CUs (about four
// waves per CU with 8-12 KiB each), and each wave's throughput is bounded by
// its own ring (loads in flight / memory latency), so the plan aims for
// roughly a thousand or more evenly loaded waves:
//  * at least two strips per CU: one single-wave workgroup per whole strip
//    (no combine at all), with about 24-32 KiB in flight per CU: ring depth
//    12 below 2.5 strips per CU, 8 up to 4, 6 up to 5.5, else 4.  Measured
//    (cold, forced depths 4/6/8/12, us): 16384 x 5120 (2 per CU) 8.96 /
//    8.05 / 7.49 / 6.94; 20480 x 5120 10.14 / 8.63 / 7.44 / 7.28; 27648 x
//    5120 (3.4) 10.86 / 8.64 / 8.19 / 8.94; 32768 x 5120 10.75 / 9.25 /
//    9.00 / 9.31; 41472 x 5120 (5.1) 12.07 / 11.81 / 12.21 / 13.05;
//    55296 x 5120 (6.75) 13.63 / 14.11 / 13.97 / 14.88; the same order at
//    K = 2560 to 6912 and up to 9 strips per CU.  At exactly 2.5 (20480 x
//    3200, a sweep shape) depths 8 and 12 tie graph-timed (5.70 / 5.66) and
//    12 was slower under the kernel trace (5.92 against 5.67), so it keeps 8;
//  * long strips (KT >= split_min_tiles): single-wave workgroups with the
//    k-range split into SG = floor(4 cus / NS) ranges (at least 2, runs of
//    at least 4 tiles), so the grid has at most 4 waves on every CU,
//    combined with one atomic per row; depth 8, or 4 for runs of at most 5
//    tiles.  Measured (cold, forced plans, us; old rule: about 3.75 waves
//    per CU rounded, depth 8 only for runs of 24 tiles or more): 12288 x
//    14336 (384 strips) 11.73 with 3 ranges against 10.21 with 2 (4.5 waves
//    on half the CUs, 3 on every CU); 6144 x 10240 6.24 at depth 4 against
//    5.31 at 8; 8192 x 6912 5.97 against 5.21; 2048 x 27648 6.01 against
//    5.14; 2560 x 6912 (runs of 5) 3.56 at 4 against 3.58 at 8;
//  * otherwise: 8-wave workgroups over whole strips, depth 4 (6 for strips of
//    40 tiles or more).
// Measured on MI355X (cold, per-launch): within 2% of the best of a sweep of
// every (waves, splits, depth) on each of the 12 workload shapes; e.g.
// 55296 x 5120 12.7 us (batch kernel 13.7), 5120 x 27648 8.1 us (8.9),
// 13824 x 2560 4.0 us (4.3), 2560 x 6912 3.58 us (3.78).
void gemv_ring_plan(const GemvPolicy &p, int64_t NS, int64_t KT, int cus, int *wk, int *sg,
                    int *run, int *depth) {
    int64_t WK = 8, SG = 1, D = KT >= 40 ? 6 : 4;
    if (NS >= 2 * int64_t(cus)) {
        WK = 1;
        // strips per CU q = NS / cus: depth 12 for q < 2.5, 8 for q <= 4,
        // 6 for q <= 5.5, else 4
        D = 2 * NS < 5 * int64_t(cus) ? 12 : NS <= 4 * int64_t(cus) ? 8
            : 2 * NS <= 11 * int64_t(cus) ? 6 : 4;
    } else if (KT >= p.split_min_tiles && KT >= 2) {
        WK = 1;
        SG = std::max<int64_t>(2, std::min<int64_t>(KT / 4, 4 * int64_t(cus) / NS));
        SG = std::min(SG, KT);
        D = ceil_div(KT, SG) <= 5 ? 4 : 8;
    }
    WK = std::min(WK, ceil_div(KT, SG));
    *wk = int(WK);
    *sg = int(SG);
    *run = int(ceil_div(ceil_div(KT, SG), WK));
    *depth = int(D);
}

namespace {

template <bool GROUPED>
hipError_t launch_ring(const GemvLaunch &la, const GemvGroups *t, int depth, hipStream_t stream) {
    if ((la.K & 15) != 0 || la.WK < 1 || la.WK > 16) return hipErrorInvalidValue;
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    GemvGroups tt = t ? *t : GemvGroups{};
    void *args[] = {&a, &tt};
    const void *fn;
#define W2A8_RING(DD)                                                                      \
    fn = GROUPED ? reinterpret_cast<const void *>(&gemv_ring_grouped_kernel<DD>)           \
                 : reinterpret_cast<const void *>(&gemv_ring_kernel<DD>)
    switch (depth) {
    case 2: W2A8_RING(2); break;
    case 4: W2A8_RING(4); break;
    case 6: W2A8_RING(6); break;
    case 8: W2A8_RING(8); break;
    case 12: W2A8_RING(12); break;
    default: return hipErrorInvalidValue;
    }
#undef W2A8_RING
    return hipLaunchKernel(fn, dim3(unsigned(a.NS), unsigned(a.SG)), dim3(unsigned(64 * a.WK)),
                           args, 0, stream);
}

}  // namespace

hipError_t launch_gemv_ring(const GemvLaunch &a, int depth, hipStream_t stream) {
    return launch_ring<false>(a, nullptr, depth, stream);
}

// Row-slice plan: the slice kernel serves matrices of small packed size
// where the ring plan would leave CUs idle or split strips.  Measured (cold,
// graph-timed, 256 CUs; time against the ring plan's):
//  * at most 4 single-wave workgroups per CU (NS <= CUs/2), strips of at
//    most 64 tiles, or 96 from NS >= CUs/4: better on every shape of N =
//    512..4096 x K = 2560..8192 (0.87-0.99, ties at N = 3840 x K <= 4096),
//    e.g. 2560 x 2560 2.74 against 2.84 us, 2560 x 6912 3.44 against 3.56,
//    4096 x 4096 3.07 against 3.22; at K = 10240-12288 from N = 2048 (3200 x
//    10240 4.01 against 4.25, 3840 x 12288 4.47 against 4.85) but not below
//    (1536 x 10240 1.01, 512 x 10240 1.03); at K = 14336 it loses below 64
//    strips (1.06-1.08); from 136 strips at K < 6144 it loses (4352 x 3200
//    1.02, 4800 x 3200 3.26 against 3.16, 6912 x 5120 1.03);
//  * up to 8 per CU (NS <= CUs) where the ring plan splits strips of 48-64
//    tiles over workgroups: 0.89-0.94 (4800 x 6912 4.02 against 4.48, 8192 x
//    8192 5.26 against 5.64), but from 80 tiles, and from 320 strips, even or
//    slower (8192 x 10240 1.01, 10240 x 8192 1.03, 12288 x 12288 1.08);
//  * at 35-71 MB far slower (5120 x 27648 9.4 against 8.3, 55296 x 5120 14.5
//    against 12.8): a strip's 8 slices are read in 128-byte pieces by 8 waves.
// Depth 4, except 6 for strips of more than 40 tiles on at most 4 workgroups
// per CU.
bool gemv_slice_plan(int64_t NS, int64_t KT, int cus, int *depth) {
    const int64_t c = cus;
    const bool take = 2 * NS <= c ? KT <= 64 || (KT <= 96 && 4 * NS >= c)
                                  : NS <= c && KT >= 48 && KT <= 64;
    if (!take) return false;
    *depth = KT > 40 && 2 * NS <= c ? 6 : 4;
    return true;
}

namespace {

template <bool GROUPED>
hipError_t launch_slice(const GemvLaunch &la, const GemvGroups *t, int depth, hipStream_t stream) {
    if ((la.K & 15) != 0 || int64_t(la.NS) * kSlices > INT32_MAX) return hipErrorInvalidValue;
    GemvLaunch a = la;
    GemvGroups tt = t ? *t : GemvGroups{};
    void *args[] = {&a, &tt};
    const void *fn;
#define W2A8_SLICE(DD)                                                                     \
    fn = GROUPED ? reinterpret_cast<const void *>(&gemv_slice_grouped_kernel<DD>)          \
                 : reinterpret_cast<const void *>(&gemv_slice_kernel<DD>)
    switch (depth) {
    case 2: W2A8_SLICE(2); break;
    case 4: W2A8_SLICE(4); break;
    case 6: W2A8_SLICE(6); break;
    case 8: W2A8_SLICE(8); break;
    default: return hipErrorInvalidValue;
    }
#undef W2A8_SLICE
    return hipLaunchKernel(fn, dim3(unsigned(a.NS) * kSlices), dim3(64), args, 0, stream);
}

}  // namespace

hipError_t launch_gemv_slice(const GemvLaunch &a, int depth, hipStream_t stream) {
    return launch_slice<false>(a, nullptr, depth, stream);
}

hipError_t launch_gemv_slice_grouped(const GemvLaunch &a, const GemvGroups &t, int depth,
                                     hipStream_t stream) {
    return launch_slice<true>(a, &t, depth, stream);
}

hipError_t launch_gemv_ring_grouped(const GemvLaunch &a, const GemvGroups &t, int depth,
                                    hipStream_t stream) {
    return launch_ring<true>(a, &t, depth, stream);
}

}  // namespace w2a8
