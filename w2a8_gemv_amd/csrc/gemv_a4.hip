// W2A4 GEMV (M = 1): ternary T32x128 weights against int4 activations (A4I
// layout, a4.h), exact int32 result.
//
// What it computes: the integer product of "如何编译 BitNet W2A8 CUDA 内核并用
// test.py 运行 GEMV 加速测试？" ("如何判断结果") with the 4-bit activations
// that "使用 BitNet 框架部署 1-bit LLM：三元权重量化、LUT 矩阵乘加速与 GPU 运行时优化",
// section "GPU 运行时优化与低延迟推理管道", names as its "a4.8" extension;
// the scale epilogue of "Windows 上跑通 BitNet b1.58：…部署实录" §3.1.
//
// Same work split, weight stream, reduction and split-k combine as the int8
// ring kernel (gemv_ring.hip): each wave keeps a ring of D weight tiles in
// flight and loads each tile's activation chunk next to it.  What changes:
//  * a tile's activations are 64 bytes (128 nibbles): a lane loads its
//    chunk as 8 bytes;
//  * decode: for each weight word, w & 0x33333333 and (w >> 2) & 0x33333333
//    put the codes c = w + 1 of 8 values each into nibbles, in the same
//    positions as their activations in the chunk's two words, so two
//    v_dot8_i32_i4 give sum c*x over 16 weights: 5 VALU per 16 weights
//    (the int8 kernel needs 9), one accumulator per row;
//  * sum_k x (for sum w*x = sum c*x - sum x) is v_dot8 against 0x11111111;
//  * A4I rows are zero-padded to 32 values, so any K takes this kernel:
//    values past K inside the row are zeros, and only chunks past the padded
//    row are clamped to a chunk inside it and counted as zero.
#include "a4.h"
#include "device.h"

namespace w2a8 {
namespace {


__device__ __forceinline__ void mac_a4(const v4u w, const v2u xv, int (&acc)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        acc[q] = dot8(v & 0x33333333u, xv[0], acc[q]);
        acc[q] = dot8((v >> 2) & 0x33333333u, xv[1], acc[q]);
    }
}

template <int D>
__global__ __launch_bounds__(1024) void gemv_a4_kernel(GemvLaunch a) {
    __shared__ int red[16 * kTileRows];
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
    const int kg = lane & 7, rg = lane >> 3;
    const int last = min(max(w0, w0 + n - 1), a.KT - 1);
    const v4u *sbase = reinterpret_cast<const v4u *>(a.wp + int64_t(s) * a.KT * kTileWords);
    // Activation chunks of 8 bytes: chunk c = 8t + kg of the padded row.
    const v2u *xp = reinterpret_cast<const v2u *>(a.x);
    const int xlast = (a.K + kA4Granule - 1) / kA4Granule * 2 - 1;   // 2 chunks per granule

    // 1. Fill the ring: tiles w0 .. w0+D-1 (clamped to `last`) and their
    //    activation chunks.
    v4u r[D];
    v2u xq[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(w0 + j, last);
        r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + lane);
        xq[j] = xp[min(t * 8 + kg, xlast)];
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. Stream: consume tile i of the run, reload its slot with tile i + D.
    int acc[4] = {0, 0, 0, 0};
    int sxl = 0;
    int i = 0;
    for (; i + D < n; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const bool in = (w0 + i + j) * 8 + kg <= xlast;
            const v2u xv = in ? xq[j] : v2u{0u, 0u};
            sxl = dot8(xv[0], 0x11111111u, dot8(xv[1], 0x11111111u, sxl));
            mac_a4(r[j], xv, acc);
            const int t = min(w0 + i + D + j, last);
            r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + lane);
            xq[j] = xp[min(t * 8 + kg, xlast)];
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < n) {
            const bool in = (w0 + i + j) * 8 + kg <= xlast;
            const v2u xv = in ? xq[j] : v2u{0u, 0u};
            sxl = dot8(xv[0], 0x11111111u, dot8(xv[1], 0x11111111u, sxl));
            mac_a4(r[j], xv, acc);
        }
    }
    const int sx = sum8(sxl);

    // 3. Reduce over the 8 lanes of a row group, then over the waves.
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rr[q] = sum8(acc[q]);
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

hipError_t launch_gemv_a4(const GemvLaunch &la, int depth, hipStream_t stream) {
    if (la.WK < 1 || la.WK > 16) return hipErrorInvalidValue;
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    void *args[] = {&a};
    const void *fn;
    switch (depth) {
    case 2: fn = reinterpret_cast<const void *>(&gemv_a4_kernel<2>); break;
    case 4: fn = reinterpret_cast<const void *>(&gemv_a4_kernel<4>); break;
    case 6: fn = reinterpret_cast<const void *>(&gemv_a4_kernel<6>); break;
    case 8: fn = reinterpret_cast<const void *>(&gemv_a4_kernel<8>); break;
    case 12: fn = reinterpret_cast<const void *>(&gemv_a4_kernel<12>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(unsigned(a.NS), unsigned(a.SG)), dim3(unsigned(64 * a.WK)),
                           args, 0, stream);
}

}  // namespace w2a8
