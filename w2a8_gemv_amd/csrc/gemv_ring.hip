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
// costs no vector instructions besides the multiply.  Activations: each wave
// stages its run into its own LDS region first (issued before the weights;
// Σx summed on the way), or, for K a multiple of 16 with DX, loads each tile's
// 16-byte chunk per lane next to the weights (a second ring).
#include "device.h"

namespace w2a8 {
namespace {

// Activation chunks (16 bytes) staged per lane: runs of at most
// kRingXChunks * 64 / 8 = 64 tiles.
constexpr int kRingXChunks = 8;

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

// IL (interleaved, with DX only): the P = SG*WK waves of a strip take its
// tiles p, p + P, p + 2P, ... (p = g*WK + wave), so the strip is read as one
// front of P adjacent tiles; otherwise each wave takes a contiguous run.
template <int D, bool DX, bool IL>
__global__ __launch_bounds__(1024) void gemv_ring_kernel(GemvLaunch a) {
    static_assert(DX || !IL, "interleaved runs load their activations directly");
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
    // Tiles of this wave: w0 + i*step, i < n.  Interleaved: KT = TQ*P + TR.
    const int p = g * a.WK + wv;
    const int w0 = IL ? p : kt0 + wv * wq + min(wv, wr);
    const int n = IL ? a.TQ + (p < a.TR ? 1 : 0) : wq + (wv < wr ? 1 : 0);
    const int step = IL ? a.SG * a.WK : 1;
    const int kg = lane & 7, rg = lane >> 3;
    // Last tile a load may touch: the run's last tile (or, for an empty run,
    // a tile of this strip).
    const int last = min(max(w0, w0 + (n - 1) * step), a.KT - 1);
    const v4u *sbase = reinterpret_cast<const v4u *>(a.wp + int64_t(s) * a.KT * kTileWords);

    uint8_t *xl = smem + wv * (a.RUN * kTileK);
    int *red = reinterpret_cast<int *>(smem + (DX ? 0 : a.WK * a.RUN * kTileK));

    // 1. Activations of the run (staged path): the 16-byte chunks that lie
    //    entirely below K, issued before the weights.
    const int kbase = w0 * kTileK;
    const int nchunk = n * (kTileK / 16);
    v4u xr[DX ? 1 : kRingXChunks];
    if constexpr (!DX) {
#pragma unroll
        for (int j = 0; j < kRingXChunks; ++j) {
            const int c = lane + 64 * j;
            xr[j] = v4u{0u, 0u, 0u, 0u};
            if (c < nchunk && kbase + 16 * c + 16 <= a.K)
                xr[j] = *reinterpret_cast<const v4u *>(a.x + kbase + 16 * c);
        }
    }

    // 2. Fill the ring: tiles w0 .. w0+D-1 (clamped to `last`).
    v4u r[D];
    v4u xq[D];   // DX: the activation ring; staged path: chunks read from LDS
    const v4u *xp = reinterpret_cast<const v4u *>(a.x);
    const int xlast = (a.K >> 4) - 1;          // last whole 16-byte chunk (DX: K % 16 == 0)
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(w0 + j * step, last);
        r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + lane);
        if constexpr (DX) xq[j] = xp[min(t * (kTileK / 16) + kg, xlast)];
        __builtin_amdgcn_sched_barrier(0);
    }

    // 3. Stage the run's activations in the wave's LDS region; sum them.
    int sx = 0;
    if constexpr (!DX) {
        if ((a.K & 15) != 0) {
            // the one chunk that straddles K, byte by byte
#pragma unroll
            for (int j = 0; j < kRingXChunks; ++j) {
                const int c = lane + 64 * j;
                const int k0 = kbase + 16 * c;
                if (c < nchunk && k0 < a.K && k0 + 16 > a.K) {
                    uint32_t b4[4] = {0u, 0u, 0u, 0u};
                    for (int i = 0; i < 16; ++i)
                        if (k0 + i < a.K) b4[i >> 2] |= uint32_t(uint8_t(a.x[k0 + i])) << (8 * (i & 3));
                    xr[j] = v4u{b4[0], b4[1], b4[2], b4[3]};
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kRingXChunks; ++j) {
            const int c = lane + 64 * j;
            if (c < nchunk) *reinterpret_cast<v4u *>(xl + 16 * c) = xr[j];
            sx = xsum16(xr[j], sx);
        }
        sx = sum8(sx);
        sx += __shfl_xor(sx, 8);
        sx += __shfl_xor(sx, 16);
        sx += __shfl_xor(sx, 32);
    }

    // 4. Stream: consume tile i of the run, reload its slot with tile i + D.
    //    Staged path: the activation chunk of each slot is read from LDS one
    //    ring ahead (right after the slot's previous use), so no tile waits
    //    for its own LDS read.
    RingAcc acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
    int sxl = 0;
    const uint8_t *xlk = xl + 16 * kg;
    const int nlast = max(n - 1, 0);
    if constexpr (!DX) {
#pragma unroll
        for (int j = 0; j < D; ++j)
            xq[j] = *reinterpret_cast<const v4u *>(xlk + min(j, nlast) * kTileK);
    }
    int i = 0;
    for (; i + D < n; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if constexpr (DX) sxl = xsum16(xq[j], sxl);
            ring_mac(r[j], xq[j], acc);
            const int t = min(w0 + (i + D + j) * step, last);
            r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + lane);
            if constexpr (DX)
                xq[j] = xp[min(t * (kTileK / 16) + kg, xlast)];
            else
                xq[j] = *reinterpret_cast<const v4u *>(xlk + min(i + D + j, nlast) * kTileK);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < n) {
            v4u xv = xq[j];
            if constexpr (DX) {
                // chunks at or past K (K % 16 == 0 here) count as zero
                const bool in = (w0 + (i + j) * step) * kTileK + 16 * kg < a.K;
                xv = in ? xv : v4u{0u, 0u, 0u, 0u};
                sxl = xsum16(xv, sxl);
            }
            ring_mac(r[j], xv, acc);
        }
    }
    if constexpr (DX) {
        // The main loop's chunks all lie below K: a run's tiles before its
        // last D are inside the strip's k-range, and only the last tile of a
        // strip can reach past K.
        sx = sum8(sxl);
    }

    // 5. Reduce: 8 lanes per row group; sum_k w*x = sum_k c*x - sum_k x over
    //    the run; then the WK waves via LDS.
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rr[q] = sum8(acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4));
    const int mine = (kg == 0 ? rr[0] : kg == 1 ? rr[1] : kg == 2 ? rr[2] : rr[3]) - sx;
    int tot = 0, r32;
    bool owner;
    int cnt = IL ? n : ntile;   // k-tiles this workgroup contributes
    if (a.WK == 1) {
        tot = mine;
        r32 = rg * 4 + kg;
        owner = kg < 4;
    } else {
        if (kg < 4) red[wv * kTileRows + rg * 4 + kg] = mine;
        if (IL && lane == 0) red[a.WK * kTileRows + wv] = n;
        __syncthreads();
        r32 = tid;
        owner = tid < kTileRows;
        if (owner)
            for (int w = 0; w < a.WK; ++w) tot += red[w * kTileRows + tid];
        if (IL) {
            cnt = 0;
            for (int w = 0; w < a.WK; ++w) cnt += red[a.WK * kTileRows + w];
        }
    }
    const int row = s * kTileRows + r32;
    const float sa = a.y_f32 ? a.sa[0] : 0.0f;
    int v = tot;
    if (a.SG > 1 && !(owner && split_add(a.ws_row + row, cnt, tot, a.KT, &v))) return;
    if (owner && row < a.N) {
        if (a.y_i32) a.y_i32[row] = v;
        if (a.y_f32) a.y_f32[row] = (float(v) * sa) * a.sw;
    }
}

// Whole strips per wave: wave w of the grid streams the consecutive strips
// [w*SQ + min(w, SR), ...) (SQ or SQ + 1 of them; NS = SQ*NW + SR), which lie
// back to back in memory, as one run through a ring of D tiles in flight,
// with each tile's activation chunk loaded next to it.  At every strip
// boundary the wave reduces its accumulators, stores the strip's 32 rows and
// starts the next strip; the ring keeps streaming meanwhile.  No cross-wave
// or cross-workgroup combine: the workgroup is only a container of WK
// independent waves.  K a multiple of 16.
template <int D>
__global__ __launch_bounds__(1024) void gemv_strips_kernel(GemvLaunch a) {
    const int lane = int(threadIdx.x) & 63;
    const int w = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * a.WK + (int(threadIdx.x) >> 6));
    if (w >= a.SG) return;                         // SG: waves in the grid
    const int s0 = w * a.KQ + min(w, a.KR);       // first strip (NS = KQ*SG + KR)
    const int nstrip = a.KQ + (w < a.KR ? 1 : 0);
    if (nstrip <= 0) return;
    const int KT = a.KT;
    const int n = nstrip * KT;
    const int last = n - 1;
    const int kg = lane & 7, rg = lane >> 3;
    const v4u *base = reinterpret_cast<const v4u *>(a.wp + int64_t(s0) * KT * kTileWords);
    const v4u *xp = reinterpret_cast<const v4u *>(a.x);
    const int xlast = (a.K >> 4) - 1;

    v4u r[D], xq[D];
    int ktn = 0;   // k-tile of the next tile to load (wraps at KT)
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(j, last);
        r[j] = __builtin_nontemporal_load(base + t * (kTileBytes / 16) + lane);
        xq[j] = xp[min(ktn * (kTileK / 16) + kg, xlast)];
        ktn = ktn + 1 == KT ? 0 : ktn + 1;
        __builtin_amdgcn_sched_barrier(0);
    }
    RingAcc acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
    int sxl = 0;
    int ktc = 0;      // k-tile of the tile being consumed
    int srow = s0 * kTileRows + rg * 4 + kg;   // this lane's row in the current strip
    const float sa = a.y_f32 ? a.sa[0] : 0.0f;
    const bool ragged = (a.K & (kTileK - 1)) != 0;

    auto consume = [&](int j) {
        v4u xv = xq[j];
        if (ragged && ktc == KT - 1) {
            // the strip's last tile reaches past K: chunks at or past K are zero
            const bool in = ktc * kTileK + 16 * kg < a.K;
            xv = in ? xv : v4u{0u, 0u, 0u, 0u};
        }
        sxl = xsum16(xv, sxl);
        ring_mac(r[j], xv, acc);
        if (ktc == KT - 1) {
            // strip boundary: reduce, store the strip's rows, restart
            int rr[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) rr[q] = sum8(acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4));
            const int v = (kg == 0 ? rr[0] : kg == 1 ? rr[1] : kg == 2 ? rr[2] : rr[3]) - sum8(sxl);
            if (kg < 4 && srow < a.N) {
                if (a.y_i32) a.y_i32[srow] = v;
                if (a.y_f32) a.y_f32[srow] = (float(v) * sa) * a.sw;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
            sxl = 0;
            srow += kTileRows;
            ktc = 0;
        } else {
            ++ktc;
        }
    };

    int i = 0;
    for (; i + D < n; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            consume(j);
            const int t = min(i + D + j, last);
            r[j] = __builtin_nontemporal_load(base + t * (kTileBytes / 16) + lane);
            xq[j] = xp[min(ktn * (kTileK / 16) + kg, xlast)];
            ktn = ktn + 1 == KT ? 0 : ktn + 1;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j)
        if (i + j < n) consume(j);
}

// Row slices: a workgroup owns 32/R rows of a strip (its slice rs of the
// tile's lane slots, R in 2, 4, 8) over a k-range, and each load instruction
// covers R consecutive tiles: lane l reads slot rs*(64/R) + l%(64/R) of tile
// t + l/(64/R).  The slots of one row group are one 128-byte line of a tile,
// so every instruction still reads whole lines (R lines of 1024/R bytes).
// Splitting rows instead of K gives as many workgroups as a k-split without
// the cross-workgroup combine.  Activations are loaded per lane next to the
// weights (each lane its own tile's chunk; K a multiple of 16).  Lanes past
// the run's last tile load a tile inside it and use zero activations.
template <int D, int R>
__global__ __launch_bounds__(1024) void gemv_rows_slice_kernel(GemvLaunch a) {
    constexpr int L = 64 / R;                     // lanes per tile segment
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int *red = reinterpret_cast<int *>(smem);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = int(blockIdx.x) / R;
    const int rs = int(blockIdx.x) % R;
    const int g = int(blockIdx.y);
    const bool big = g < a.KR;
    const int kt0 = g * a.KQ + min(g, a.KR);
    const int ntile = a.KQ + (big ? 1 : 0);
    const int wq = big ? a.WQ1 : a.WQ0, wr = big ? a.WR1 : a.WR0;
    const int w0 = kt0 + wv * wq + min(wv, wr);
    const int n = wq + (wv < wr ? 1 : 0);
    const int u = lane / L;                      // tile offset of this lane
    const int slot = rs * L + lane % L;          // lane slot within the tile
    const int kg = slot & 7, rgl = (lane % L) >> 3;   // rgl: row group within the slice
    const int ni = (n + R - 1) / R;              // load instructions of the run
    const int lastt = max(w0 + n - 1, w0);       // last tile of the run (a valid address)
    const v4u *sbase = reinterpret_cast<const v4u *>(a.wp + int64_t(s) * a.KT * kTileWords);
    const v4u *xp = reinterpret_cast<const v4u *>(a.x);
    const int xlast = (a.K >> 4) - 1;

    v4u r[D], xq[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(w0 + j * R + u, lastt);
        r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + slot);
        xq[j] = xp[min(t * (kTileK / 16) + kg, xlast)];
        __builtin_amdgcn_sched_barrier(0);
    }
    RingAcc acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
    int sxl = 0;
    int i = 0;
    for (; i + D < ni; i += D) {
        // instructions before the run's last D cover whole groups of R tiles
        // that lie below K (only the strip's last tile reaches past K)
#pragma unroll
        for (int j = 0; j < D; ++j) {
            sxl = xsum16(xq[j], sxl);
            ring_mac(r[j], xq[j], acc);
            const int t = min(w0 + (i + D + j) * R + u, lastt);
            r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + slot);
            xq[j] = xp[min(t * (kTileK / 16) + kg, xlast)];
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < ni) {
            const int tt = (i + j) * R + u;      // tile of this lane within the run
            const bool in = tt < n && (w0 + tt) * kTileK + 16 * kg < a.K;
            const v4u xv = in ? xq[j] : v4u{0u, 0u, 0u, 0u};
            sxl = xsum16(xv, sxl);
            ring_mac(r[j], xv, acc);
        }
    }
    // Per row q of this lane's row group: sum_k c*x - sum_k x over the lane's
    // chunks, then summed over kg (8 lanes) and over the R tile offsets.
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int v = sum8(acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4) - sxl);
#pragma unroll
        for (int o = L; o < 64; o <<= 1) v += __shfl_xor(v, o);
        rr[q] = v;
    }
    constexpr int RW = kTileRows / R;            // rows of the slice
    const int mine = kg == 0 ? rr[0] : kg == 1 ? rr[1] : kg == 2 ? rr[2] : rr[3];
    int tot = 0, rloc;
    bool owner;
    if (a.WK == 1) {
        tot = mine;
        rloc = rgl * 4 + kg;
        owner = u == 0 && kg < 4;
    } else {
        if (u == 0 && kg < 4) red[wv * RW + rgl * 4 + kg] = mine;
        __syncthreads();
        rloc = tid;
        owner = tid < RW;
        if (owner)
            for (int w = 0; w < a.WK; ++w) tot += red[w * RW + tid];
    }
    const int row = s * kTileRows + rs * RW + rloc;
    const float sa = a.y_f32 ? a.sa[0] : 0.0f;
    int v = tot;
    if (a.SG > 1 && !(owner && split_add(a.ws_row + row, ntile, tot, a.KT, &v))) return;
    if (owner && row < a.N) {
        if (a.y_i32) a.y_i32[row] = v;
        if (a.y_f32) a.y_f32[row] = (float(v) * sa) * a.sw;
    }
}

}  // namespace

// LDS of the ring kernel: per-wave activation regions of RUN tiles (staged
// path) and the row partials.
size_t gemv_ring_lds_bytes(const GemvLaunch &a, bool dx) {
    // (+ one tile count per wave for interleaved runs)
    return (dx ? 0 : size_t(a.WK) * a.RUN * kTileK) + size_t(a.WK) * (kTileRows + 1) * 4;
}

bool gemv_ring_fits(const GemvLaunch &a) { return a.RUN <= kRingXChunks * 8; }

hipError_t launch_gemv_ring(const GemvLaunch &la, int depth, bool dx, bool il,
                            hipStream_t stream) {
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    dx = dx && (a.K & 15) == 0;
    il = il && dx;
    a.TQ = a.KT / (a.SG * a.WK);
    a.TR = a.KT % (a.SG * a.WK);
    void *args[] = {&a};
    const void *fn;
#define W2A8_RING(DD)                                                                         \
    fn = il   ? reinterpret_cast<const void *>(&gemv_ring_kernel<DD, true, true>)             \
         : dx ? reinterpret_cast<const void *>(&gemv_ring_kernel<DD, true, false>)            \
              : reinterpret_cast<const void *>(&gemv_ring_kernel<DD, false, false>)
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
                           args, gemv_ring_lds_bytes(a, dx), stream);
}

hipError_t launch_gemv_rows_slice(const GemvLaunch &la, int depth, int slices,
                                  hipStream_t stream) {
    if ((la.K & 15) != 0) return hipErrorInvalidValue;
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    void *args[] = {&a};
    const void *fn = nullptr;
#define W2A8_SLICE(DD, RR)                                                                    \
    if (depth == DD && slices == RR) fn = reinterpret_cast<const void *>(&gemv_rows_slice_kernel<DD, RR>)
    W2A8_SLICE(4, 2); W2A8_SLICE(8, 2); W2A8_SLICE(12, 2);
    W2A8_SLICE(4, 4); W2A8_SLICE(8, 4); W2A8_SLICE(12, 4);
    W2A8_SLICE(4, 8); W2A8_SLICE(8, 8); W2A8_SLICE(12, 8);
    W2A8_SLICE(6, 2); W2A8_SLICE(6, 4); W2A8_SLICE(6, 8);
#undef W2A8_SLICE
    if (!fn) return hipErrorInvalidValue;
    return hipLaunchKernel(fn, dim3(unsigned(a.NS * slices), unsigned(a.SG)),
                           dim3(unsigned(64 * a.WK)), args,
                           size_t(a.WK) * (kTileRows / slices) * 4, stream);
}

hipError_t launch_gemv_strips(const GemvLaunch &la, int depth, int strips_per_wave,
                              hipStream_t stream) {
    if ((la.K & 15) != 0 || strips_per_wave < 1) return hipErrorInvalidValue;
    GemvLaunch a = la;
    const int nw = int(ceil_div(a.NS, strips_per_wave));    // waves in the grid
    a.SG = nw;
    a.KQ = a.NS / nw;
    a.KR = a.NS % nw;
    a.TQ = a.TR = 0;
    void *args[] = {&a};
    const void *fn;
    switch (depth) {
    case 2: fn = reinterpret_cast<const void *>(&gemv_strips_kernel<2>); break;
    case 4: fn = reinterpret_cast<const void *>(&gemv_strips_kernel<4>); break;
    case 6: fn = reinterpret_cast<const void *>(&gemv_strips_kernel<6>); break;
    case 8: fn = reinterpret_cast<const void *>(&gemv_strips_kernel<8>); break;
    case 12: fn = reinterpret_cast<const void *>(&gemv_strips_kernel<12>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(unsigned(ceil_div(nw, a.WK))), dim3(unsigned(64 * a.WK)), args,
                           0, stream);
}

}  // namespace w2a8
