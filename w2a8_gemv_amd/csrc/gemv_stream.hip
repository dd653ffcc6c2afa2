// W2A8 GEMV (M = 1), streaming variant for large matrices (gfx950).
//
// Computes exactly what gemv.hip computes — the integer product of int8
// activations and ternary weights ("如何编译 BitNet W2A8 CUDA 内核并用 test.py
// 运行 GEMV 加速测试？", sections "运行 test.py 做 GEMV 基准测试" and "如何判断结果")
// with the scale epilogue of "Windows 上跑通 BitNet b1.58：…部署实录" §3.1 —
// with a launch shaped for bandwidth rather than latency:
//
//  * A fixed grid of G long-lived waves.  The packed matrix is one linear
//    sequence of 1 KiB tiles (strip-major, which is also memory order); wave
//    w streams the contiguous tiles [w*T/G, (w+1)*T/G) across strip
//    boundaries with two load batches of U tiles in flight.
//  * Each workgroup stages all K activations once in LDS (zero past K), plus
//    one zero row that masked tiles of a batch read.
//  * Decode and dot products as in gemv.hip (codes c = w+1 masked into
//    scale-1/4/16 bytes, v_dot4_i32_i8, sum w*x = sum c*x - sum x); each lane
//    also sums its activation bytes, so sum x over a segment needs no table.
//  * Batches never cross a strip, and every tile of a batch is consumed, so
//    the loop body has no load-dependent branch and its one exit is at the
//    bottom: the compiler's wait counts then track exactly the batch being
//    multiplied.
//  * At the end of a strip segment the 8 lanes of each row group are summed
//    with DPP.  A segment that is a whole strip stores y directly.  A
//    segment that is part of a strip (at most the first and the last of a
//    wave) is combined after the stream with one device-scope atomic per row
//    (split_add in common.h); the last contributor of a row stores it.
//
// Off by default: on gfx950 the workgroup kernel is as fast or faster on the
// measured shapes (the end-of-stream atomic round trip and the per-workgroup
// staging of all of K are fixed costs this kernel pays).
#include "device.h"

namespace w2a8 {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 64 * kWavesPerBlock;
// Activation chunks (16 bytes) each thread stages: K <= kStageChunks*16*256.
constexpr int kStageChunks = 8;

struct Acc {
    int a1[4], a4[4], a16[4];
    int sx;   // sum of this lane's activation bytes over the segment
};

__device__ __forceinline__ void acc_zero(Acc &acc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
    acc.sx = 0;
}

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
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.sx = dot4(xv[j], 0x01010101u, acc.sx);
}

// Row value owned by this lane (rows 4rg + kg for kg < 4) of a finished
// segment: sum_k c*x - sum_k x over the segment, reduced over the row group.
__device__ __forceinline__ int row_value(const Acc &acc, int kg) {
    int r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = sum8(acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4));
    return (kg == 0 ? r[0] : kg == 1 ? r[1] : kg == 2 ? r[2] : r[3]) - sum8(acc.sx);
}

__device__ __forceinline__ void store_out(const GemvLaunch &a, float sa, int row, int v) {
    if (a.y_i32) a.y_i32[row] = v;
    if (a.y_f32) a.y_f32[row] = (float(v) * sa) * a.sw;
}

// U loads of tiles start..start+U-1, clamped to `last`.
template <int U>
__device__ __forceinline__ void load_batch(const v4u *wt, int start, int last, v4u (&w)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        w[u] = __builtin_nontemporal_load(wt + int64_t(min(start + u, last)) * (kTileBytes / 16));
    __builtin_amdgcn_sched_barrier(0);
}

// Multiply the first `len` tiles of a batch; kt0 is the k-tile of its first.
// Every tile is consumed (the rest read the zeroed activation row at
// `zrow`), so no load of the batch is left pending past this point.
template <int U>
__device__ __forceinline__ void mac_batch(const v4u (&w)[U], const uint8_t *xl, int kt0, int len,
                                          int zrow, int kg, Acc &acc) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int row = u < len ? kt0 + u : zrow;
        const v4u xv = *reinterpret_cast<const v4u *>(xl + row * kTileK + 16 * kg);
        mac(w[u], xv, acc);
    }
}

// A partial strip segment waiting to be added to the workspace.
struct Partial {
    int strip;    // -1: none
    int tiles;    // tiles contributed
    int val;      // this lane's row value (lanes with kg < 4)
};

template <int U>
__global__ __launch_bounds__(kThreads) void gemv_stream_kernel(GemvLaunch a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = int(blockIdx.x) * kWavesPerBlock + wv;
    const int KT = a.KT;
    const int kg = lane & 7, rg = lane >> 3;

    uint8_t *xl = smem;   // KT rows of 128 activations, then a zero row

    // This wave's tile range (empty for the grid's spare waves).
    int t0 = 0, t1 = 0;
    if (wave < a.G) {
        t0 = wave * a.TQ + min(wave, a.TR);
        t1 = t0 + a.TQ + (wave < a.TR ? 1 : 0);
    }
    const bool busy = t1 > t0;

    // 1. Activation chunks into registers first, with unconditional loads of
    //    a clamped chunk (K >= 16, so chunk 0 always lies below K); chunks at
    //    or past K are zeroed when staged.
    const int nchunk = KT * (kTileK / 16);
    const int cfull = a.K / 16;                   // chunks entirely below K
    v4u xr[kStageChunks];
#pragma unroll
    for (int j = 0; j < kStageChunks; ++j) {
        const int c = min(tid + j * kThreads, cfull - 1);
        xr[j] = *reinterpret_cast<const v4u *>(a.x + 16 * c);
    }

    // 2. The first two weight batches.  Batches never cross a strip: the
    //    load cursor `ln` advances through segments ending at `lend`.
    const v4u *wt = reinterpret_cast<const v4u *>(a.wp) + lane;
    const int last = busy ? t1 - 1 : 0;
    int ln = t0, lend = busy ? min(t1, (t0 / KT + 1) * KT) : t0;
    auto next_batch = [&](int &bs, int &bn) {
        bs = ln;
        bn = min(U, lend - ln);
        ln += bn;
        if (ln == lend) lend = min(t1, lend + KT);
    };
    int xs, xn, ys, yn;
    next_batch(xs, xn);
    next_batch(ys, yn);
    v4u wx[U], wy[U];
    // Unconditional (a spare wave reads tile 0), so the wait counts that
    // follow stay exact.
    load_batch<U>(wt, xs, last, wx);
    load_batch<U>(wt, ys, last, wy);

    // 3. Stage activations in LDS (the chunk straddling K, when K % 16 != 0,
    //    assembled byte by byte; zero past K) and the zero row.
#pragma unroll
    for (int j = 0; j < kStageChunks; ++j) {
        const int c = tid + j * kThreads;
        v4u v = c < cfull ? xr[j] : v4u{0u, 0u, 0u, 0u};
        if (c == cfull && (a.K & 15) != 0) {
            uint32_t b4[4] = {0u, 0u, 0u, 0u};
            for (int i = 0; i < (a.K & 15); ++i)
                b4[i >> 2] |= uint32_t(uint8_t(a.x[16 * c + i])) << (8 * (i & 3));
            v = v4u{b4[0], b4[1], b4[2], b4[3]};
        }
        if (c < nchunk) *reinterpret_cast<v4u *>(xl + 16 * c) = v;
    }
    if (tid < 8) *reinterpret_cast<v4u *>(xl + KT * kTileK + 16 * tid) = v4u{0u, 0u, 0u, 0u};
    __syncthreads();
    if (!busy) return;

    // 4. Stream.  At a strip segment's end (`cend`) the row values are
    //    stored (whole strip) or kept (part of a strip).
    const float sa = a.y_f32 ? a.sa[0] : 0.0f;
    Acc acc;
    acc_zero(acc);
    int seg_s = t0 / KT, seg_base = seg_s * KT, seg_k0 = t0 - seg_base;
    int cend = min(t1, seg_base + KT);
    Partial p0 = {-1, 0, 0}, p1 = {-1, 0, 0};

    auto finish = [&](int t_end) {
        if (t_end != cend) return;                    // segment continues
        const int k_end = t_end - seg_base;
        const int v = row_value(acc, kg);
        const int row = seg_s * kTileRows + rg * 4 + kg;
        if (seg_k0 == 0 && k_end == KT) {
            if (kg < 4 && row < a.N) store_out(a, sa, row, v);
        } else if (p0.strip < 0) {
            p0 = {seg_s, k_end - seg_k0, v};
        } else {
            p1 = {seg_s, k_end - seg_k0, v};
        }
        acc_zero(acc);
        seg_s += 1;
        seg_base += KT;
        seg_k0 = 0;
        cend = min(t1, cend + KT);
    };

    // One exit, at the bottom: the loop head is reached with batch X issued
    // before batch Y on every path, which keeps its wait counts exact.  An
    // empty Y batch (the range ended with X) is consumed as masked tiles.
    while (true) {
        mac_batch<U>(wx, xl, xs - seg_base, xn, KT, kg, acc);
        finish(xs + xn);
        next_batch(xs, xn);
        load_batch<U>(wt, xs, last, wx);
        mac_batch<U>(wy, xl, ys - seg_base, yn, KT, kg, acc);
        if (yn > 0) finish(ys + yn);
        next_batch(ys, yn);
        load_batch<U>(wt, ys, last, wy);
        if (xn == 0) break;
    }

    // 5. Partial strips: one device-scope atomic per row combines them (both
    //    of a wave's partials in flight together); the last contributor of a
    //    row stores it.
    if (p0.strip < 0 || kg >= 4) return;
    const int r0 = p0.strip * kTileRows + rg * 4 + kg;
    int v;
    if (p1.strip < 0) {
        if (split_add(a.ws_row + r0, p0.tiles, p0.val, KT, &v) && r0 < a.N) store_out(a, sa, r0, v);
        return;
    }
    const int r1 = p1.strip * kTileRows + rg * 4 + kg;
    const uint64_t add0 = split_word(p0.tiles, p0.val), add1 = split_word(p1.tiles, p1.val);
    const uint64_t t0w =
        __hip_atomic_fetch_add(a.ws_row + r0, add0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t1w =
        __hip_atomic_fetch_add(a.ws_row + r1, add1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (split_done(a.ws_row + r0, t0w + add0, KT, &v) && r0 < a.N) store_out(a, sa, r0, v);
    if (split_done(a.ws_row + r1, t1w + add1, KT, &v) && r1 < a.N) store_out(a, sa, r1, v);
}

}  // namespace

size_t gemv_stream_lds_bytes(const GemvLaunch &a) {
    return size_t(a.KT + 1) * kTileK;
}

bool gemv_stream_fits(int64_t K) {
    const int64_t KT = (K + kTileK - 1) / kTileK;
    return K >= 16 && KT * (kTileK / 16) <= int64_t(kStageChunks) * kThreads;
}

hipError_t launch_gemv_stream(const GemvLaunch &la, hipStream_t stream) {
    GemvLaunch a = la;
    const int64_t T = int64_t(a.NS) * a.KT;
    a.TQ = int(T / a.G);
    a.TR = int(T % a.G);
    const unsigned blocks = unsigned((a.G + kWavesPerBlock - 1) / kWavesPerBlock);
    void *args[] = {&a};
    const void *fn;
    switch (a.unroll) {
    case 2: fn = reinterpret_cast<const void *>(&gemv_stream_kernel<2>); break;
    case 8: fn = reinterpret_cast<const void *>(&gemv_stream_kernel<8>); break;
    default: fn = reinterpret_cast<const void *>(&gemv_stream_kernel<4>); break;
    }
    return hipLaunchKernel(fn, dim3(blocks), dim3(kThreads), args, gemv_stream_lds_bytes(a),
                           stream);
}

}  // namespace w2a8
