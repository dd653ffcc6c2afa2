// W2A4 GEMV (M = 1): ternary T32x128 weights against int4 activations (A4I
// layout, a4.h), exact int32 result.
//
// What it computes: the integer product of "如何编译 BitNet W2A8 CUDA 内核并用
// test.py 运行 GEMV 加速测试？" ("如何判断结果") with the 4-bit activations
// that "使用 BitNet 框架部署 1-bit LLM：三元权重量化、LUT 矩阵乘加速与 GPU 运行时优化",
// section "GPU 运行时优化与低延迟推理管道", names as its "a4.8" extension;
// the scale epilogue of "Windows 上跑通 BitNet b1.58：…部署实录" §3.1.
//
// Same work split, loads, staging, reduction and split-k combine as the
// int8 workgroup kernel (gemv.hip); what changes:
//  * a tile's activations are 64 bytes (128 nibbles) and a lane reads its
//    chunk as 8 bytes from the wave's LDS region;
//  * decode: for each weight word, w & 0x33333333 and (w >> 2) & 0x33333333
//    put the codes c = w + 1 of 8 values each into nibbles, in the same
//    positions as their activations in the chunk's two words, so two
//    v_dot8_i32_i4 give sum c*x over 16 weights: 5 VALU per 16 weights
//    (the int8 kernel needs 9), one accumulator per row;
//  * sum_k x (for sum w*x = sum c*x - sum x) is v_dot8 against 0x11111111.
#include "a4.h"
#include "device.h"

namespace w2a8 {
namespace {


constexpr int kA4TileBytes = kTileK / 2;   // activation bytes per k-tile (64)
// Activation granules (16 bytes, 2 chunks) staged per lane: runs of at most
// 32 tiles = 128 granules.
constexpr int kA4Granules = 2;


__device__ __forceinline__ void mac_a4(const v4u w, const v2u xv, int (&acc)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        acc[q] = dot8(v & 0x33333333u, xv[0], acc[q]);
        acc[q] = dot8((v >> 2) & 0x33333333u, xv[1], acc[q]);
    }
}

template <int U>
__device__ __forceinline__ void mac_batch(const v4u (&w)[U], const uint8_t *xl, int n, int b,
                                          int kg, int (&acc)[4]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (b * U + u < n) {
            const v2u xv =
                *reinterpret_cast<const v2u *>(xl + (b * U + u) * kA4TileBytes + 8 * kg);
            mac_a4(w[u], xv, acc);
        }
    }
}

template <int U>
__global__ __launch_bounds__(1024) void gemv_a4_kernel(GemvLaunch a) {
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

    // LDS: per-wave activation regions of RUN tiles, then the row partials.
    uint8_t *xl = smem + wv * (a.RUN * kA4TileBytes);
    int *red = reinterpret_cast<int *>(smem + a.WK * a.RUN * kA4TileBytes);

    const v4u *wt = reinterpret_cast<const v4u *>(a.wp + int64_t(s) * a.KT * kTileWords) + lane;
    const int last = min(max(w0, w1 - 1), a.KT - 1);

    // 1. The run's activation granules that exist in the padded row, loaded
    //    before the weights (granules past the row read as zero).
    const uint8_t *xg = reinterpret_cast<const uint8_t *>(a.x);
    const int gbase = w0 * (kTileK / kA4Granule);
    const int ngran = n * (kTileK / kA4Granule);
    const int grow = (a.K + kA4Granule - 1) / kA4Granule;
    v4u xr[kA4Granules];
#pragma unroll
    for (int j = 0; j < kA4Granules; ++j) {
        const int c = lane + 64 * j;
        xr[j] = v4u{0u, 0u, 0u, 0u};
        if (c < ngran && gbase + c < grow)
            xr[j] = *reinterpret_cast<const v4u *>(xg + 16 * (gbase + c));
    }

    // 2. Two batches of weight loads in flight (clamped to the run).
    v4u wa[U], wb[U];
    load_batch<U>(wt, w0, last, 0, wa);
    load_batch<U>(wt, w0, last, 1, wb);

    // 3. Stage the run's activations and sum them.
    int sx = 0;
#pragma unroll
    for (int j = 0; j < kA4Granules; ++j) {
        const int c = lane + 64 * j;
        if (c < ngran) *reinterpret_cast<v4u *>(xl + 16 * c) = xr[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) sx = dot8(xr[j][e], 0x11111111u, sx);
    }
    sx = sum8(sx);
    sx += __shfl_xor(sx, 8);
    sx += __shfl_xor(sx, 16);
    sx += __shfl_xor(sx, 32);

    // 4. Stream the run: multiply one batch while the next is in flight.
    int acc[4] = {0, 0, 0, 0};
    if (n > 0) {
        int b = 0;
        for (; b + 2 < nb; b += 2) {
            mac_batch<U>(wa, xl, n, b, kg, acc);
            load_batch<U>(wt, w0, last, b + 2, wa);
            mac_batch<U>(wb, xl, n, b + 1, kg, acc);
            load_batch<U>(wt, w0, last, b + 3, wb);
        }
        mac_batch<U>(wa, xl, n, b, kg, acc);
        if (b + 1 < nb) mac_batch<U>(wb, xl, n, b + 1, kg, acc);
    }

    // 5. Reduce over the 8 lanes of a row group, then over the waves.
    int r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = sum8(acc[q]);
    const int mine = (kg == 0 ? r[0] : kg == 1 ? r[1] : kg == 2 ? r[2] : r[3]) - sx;
    int tot = 0;
    int r32;
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
    const int row = s * kTileRows + r32;
    const float sa = a.y_f32 ? a.sa[0] : 0.0f;
    int v = tot;
    if (a.SG > 1 && !(owner && split_add(a.ws_row + row, ntile, tot, a.KT, &v))) return;
    if (owner && row < a.N) {
        if (a.y_i32) a.y_i32[row] = v;
        if (a.y_f32) a.y_f32[row] = (float(v) * sa) * a.sw;
    }
}

}  // namespace

hipError_t launch_gemv_a4(const GemvLaunch &la, hipStream_t stream) {
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    void *args[] = {&a};
    const void *fn = a.unroll == 2   ? reinterpret_cast<const void *>(&gemv_a4_kernel<2>)
                     : a.unroll == 4 ? reinterpret_cast<const void *>(&gemv_a4_kernel<4>)
                                     : reinterpret_cast<const void *>(&gemv_a4_kernel<8>);
    const size_t lds = size_t(a.WK) * a.RUN * kA4TileBytes + size_t(a.WK) * kTileRows * 4;
    return hipLaunchKernel(fn, dim3(unsigned(a.NS), unsigned(a.SG)), dim3(unsigned(64 * a.WK)),
                           args, lds, stream);
}

}  // namespace w2a8
