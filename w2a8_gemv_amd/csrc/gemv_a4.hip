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

__device__ __forceinline__ float absmax8(float m, const v4u v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(lo_bf16(v[i])), fabsf(hi_bf16(v[i]))));
    return m;
}

// FUSED: the activations arrive as the bf16 row (a.xb).  Before the weight
// ring, each thread loads the first part of its share of the row for the
// maximum and the first 16-value chunk it will quantize (L2 hits that then
// need not wait behind the weights).  After the ring is in flight the
// workgroup takes the row maximum (DPP within waves, LDS across them) and
// quantizes its runs' chunks into LDS in the A4I layout (values past K as
// zeros) with the quantizer's element function (q4, a4.h).  The stream then
// reads each tile's chunk from LDS, and the epilogue uses the scale computed
// here.
// MS (fused only): the waves of a workgroup take a.WK consecutive strips
// over one k-range (one wave per strip), and quantize that k-range once into
// one LDS region they all read: the row's maximum and quantization are
// shared by a.WK strips instead of being redone for each.
template <int D, bool FUSED, bool MS>
__device__ __forceinline__ void a4_body(const GemvLaunch &a) {
    __shared__ int red[16 * kTileRows];
    __shared__ __attribute__((aligned(16))) float wmax[16];
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = MS ? int(blockIdx.x) * a.WK + wv : int(blockIdx.x);
    const bool live = !MS || s < a.NS;
    const int g = int(blockIdx.y);
    const bool big = g < a.KR;
    const int kt0 = g * a.KQ + min(g, a.KR);
    const int ntile = a.KQ + (big ? 1 : 0);
    const int wq = big ? a.WQ1 : a.WQ0, wr = big ? a.WR1 : a.WR0;
    // Tiles of this wave: w0 .. w0+n-1; loads past the run re-read its last
    // tile (an empty run: a tile of this strip).
    const int w0 = MS ? kt0 : kt0 + wv * wq + min(wv, wr);
    const int n = MS ? ntile : wq + (wv < wr ? 1 : 0);
    const int kg = lane & 7, rg = lane >> 3;
    const int last = min(max(w0, w0 + n - 1), a.KT - 1);
    const v4u *sbase =
        reinterpret_cast<const v4u *>(a.wp + int64_t(MS ? min(s, a.NS - 1) : s) * a.KT * kTileWords);
    // Activation chunks of 8 bytes: chunk c = 8t + kg of the padded row.
    const v2u *xp = reinterpret_cast<const v2u *>(a.x);
    const int xlast = (a.K + kA4Granule - 1) / kA4Granule * 2 - 1;   // 2 chunks per granule

    // 0. Fused: the first share of the row maximum and the first chunk to
    //    quantize (chunk c of the run holds values 16(8 w0 + c) .. +15).
    const int K = a.K;
    const int bd = int(blockDim.x);
    const v4u *r8 = reinterpret_cast<const v4u *>(a.xb);
    const int qfirst = MS ? tid : lane, qstride = MS ? bd : 64;
    v4u mx0 = {0u, 0u, 0u, 0u}, mx1 = {0u, 0u, 0u, 0u}, qa = {0u, 0u, 0u, 0u}, qb = qa;
    bool qpre = false;
    if constexpr (FUSED) {
        if (tid < (K >> 3)) mx0 = r8[tid];
        if (tid + bd < (K >> 3)) mx1 = r8[tid + bd];
        qpre = qfirst < 8 * n && 16 * (8 * w0 + qfirst) + 16 <= K;
        if (qpre) {
            const v4u *p = reinterpret_cast<const v4u *>(a.xb + 16 * (8 * w0 + qfirst));
            qa = p[0];
            qb = p[1];
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // 1. Fill the ring: tiles w0 .. w0+D-1 (clamped to `last`) and, unless
    //    fused, their activation chunks.
    v4u r[D];
    v2u xq[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(w0 + j, last);
        r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + lane);
        if constexpr (!FUSED) xq[j] = xp[min(t * 8 + kg, xlast)];
        __builtin_amdgcn_sched_barrier(0);
    }

    float sa = 0.0f;
    const v2u *xl = nullptr;   // fused: the run's quantized chunks in LDS
    if constexpr (FUSED) {
        // Row maximum over the workgroup (a zero chunk adds nothing).
        float amax = absmax8(absmax8(0.0f, mx0), mx1);
        int c = tid + 2 * bd;
        for (; c + 3 * bd < (K >> 3); c += 4 * bd) {   // four loads in flight
            const v4u v0 = r8[c], v1 = r8[c + bd], v2 = r8[c + 2 * bd], v3 = r8[c + 3 * bd];
            amax = absmax8(absmax8(absmax8(absmax8(amax, v0), v1), v2), v3);
        }
        for (; c < (K >> 3); c += bd) amax = absmax8(amax, r8[c]);
        if (tid == 0)
            for (int k = K & ~7; k < K; ++k)
                amax = fmaxf(amax, fabsf(__uint_as_float(uint32_t(a.xb[k]) << 16)));
        amax = wave_max_nonneg(amax);
        if (lane == 0) wmax[wv] = amax;
        if (tid >= a.WK && tid < 16) wmax[tid] = 0.0f;
        __syncthreads();
        {
            const v4u *w4 = reinterpret_cast<const v4u *>(wmax);
            const v4u q0 = w4[0], q1 = w4[1], q2 = w4[2], q3 = w4[3];
            float m4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m4[i] = fmaxf(fmaxf(__uint_as_float(q0[i]), __uint_as_float(q1[i])),
                              fmaxf(__uint_as_float(q2[i]), __uint_as_float(q3[i])));
            amax = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        }
        // The quantizer's reciprocal and scale; a zero row quantizes to 0.
        const float inv = amax == 0.0f ? 0.0f : fminf(7.0f / amax, __FLT_MAX__);
        sa = amax / 7.0f;
        v2u *region = reinterpret_cast<v2u *>(MS ? smem : smem + wv * (a.RUN * 64));
        for (int c = qfirst; c < 8 * n; c += qstride) {
            const int k0 = 16 * (8 * w0 + c);
            float v[16];
            if (k0 + 16 <= K) {
                v4u lo = qa, hi = qb;
                if (!(qpre && c == qfirst)) {
                    const v4u *p = reinterpret_cast<const v4u *>(a.xb + k0);
                    lo = p[0];
                    hi = p[1];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = lo_bf16(lo[j]);
                    v[2 * j + 1] = hi_bf16(lo[j]);
                    v[8 + 2 * j] = lo_bf16(hi[j]);
                    v[8 + 2 * j + 1] = hi_bf16(hi[j]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[i] = k0 + i < K ? __uint_as_float(uint32_t(a.xb[k0 + i]) << 16) : 0.0f;
            }
            uint32_t q0, q1;
            chunk_a4(v, inv, q0, q1);
            region[c] = v2u{q0, q1};
        }
        if constexpr (MS) {
            __syncthreads();
        } else {
            // The run is read back by other lanes of the same wave: LDS
            // accesses of a wave complete in order; keep the compiler from
            // moving them.
            __builtin_amdgcn_wave_barrier();
        }
        xl = region;
    }

    // 2. Stream: consume tile i of the run, reload its slot with tile i + D.
    const int ns = live ? n : 0;
    int acc[4] = {0, 0, 0, 0};
    int sxl = 0;
    int i = 0;
    for (; i + D < ns; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            v2u xv;
            if constexpr (FUSED) {
                xv = xl[(i + j) * 8 + kg];
            } else {
                const bool in = (w0 + i + j) * 8 + kg <= xlast;
                xv = in ? xq[j] : v2u{0u, 0u};
            }
            sxl = dot8(xv[0], 0x11111111u, dot8(xv[1], 0x11111111u, sxl));
            mac_a4(r[j], xv, acc);
            const int t = min(w0 + i + D + j, last);
            r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + lane);
            if constexpr (!FUSED) xq[j] = xp[min(t * 8 + kg, xlast)];
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < ns) {
            v2u xv;
            if constexpr (FUSED) {
                xv = xl[(i + j) * 8 + kg];
            } else {
                const bool in = (w0 + i + j) * 8 + kg <= xlast;
                xv = in ? xq[j] : v2u{0u, 0u};
            }
            sxl = dot8(xv[0], 0x11111111u, dot8(xv[1], 0x11111111u, sxl));
            mac_a4(r[j], xv, acc);
        }
    }
    const int sx = sum8(sxl);

    // 3. Reduce over the 8 lanes of a row group, then over the waves of the
    //    strip.
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rr[q] = sum8(acc[q]);
    const int mine = (kg == 0 ? rr[0] : kg == 1 ? rr[1] : kg == 2 ? rr[2] : rr[3]) - sx;
    int tot = 0, r32;
    bool owner;
    if (MS || a.WK == 1) {
        tot = mine;
        r32 = rg * 4 + kg;
        owner = live && kg < 4;
    } else {
        if (kg < 4) red[wv * kTileRows + rg * 4 + kg] = mine;
        __syncthreads();
        r32 = tid;
        owner = tid < kTileRows;
        if (owner)
            for (int w = 0; w < a.WK; ++w) tot += red[w * kTileRows + tid];
    }
    const int row = s * kTileRows + r32;
    if constexpr (!FUSED) sa = a.y_f32 ? a.sa[0] : 0.0f;
    int v = tot;
    if (a.SG > 1 && !(owner && split_add(a.ws_row + row, ntile, tot, a.KT, &v))) return;
    if (owner && row < a.N) {
        if (a.y_i32) a.y_i32[row] = v;
        if (a.y_f32) a.y_f32[row] = (float(v) * sa) * a.sw;
    }
}

template <int D>
__global__ __launch_bounds__(1024) void gemv_a4_kernel(GemvLaunch a) {
    a4_body<D, false, false>(a);
}

// Row-slice form for matrices of few strips, as the int8 row-slice kernel
// (gemv_ring.hip): workgroup (s, sl) owns row group sl (4 rows) of every tile
// of strip s; a step reads the 128-byte slice of 8 consecutive tiles (lane l:
// tile l/8 of the step, chunk l%8) and its 8-byte activation chunks.  No
// split: a row's value is the sum over the whole wave.
template <int D>
__global__ __launch_bounds__(64) void gemv_a4_slice_kernel(GemvLaunch a) {
    const int lane = threadIdx.x;
    const int s = int(blockIdx.x) / 8, sl = int(blockIdx.x) % 8;
    const int u = lane >> 3, kg = lane & 7;
    const int off = sl * 8 + kg;
    const int nst = (a.KT + 7) / 8;
    const int last = a.KT - 1;
    const v4u *sbase = reinterpret_cast<const v4u *>(a.wp + int64_t(s) * a.KT * kTileWords);
    const v2u *xp = reinterpret_cast<const v2u *>(a.x);
    const int xlast = (a.K + kA4Granule - 1) / kA4Granule * 2 - 1;   // 2 chunks per granule

    v4u r[D];
    v2u xq[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int t = min(j * 8 + u, last);
        r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + off);
        xq[j] = xp[min(t * 8 + kg, xlast)];
        __builtin_amdgcn_sched_barrier(0);
    }
    // Every step but the last holds tiles before the strip's last one, whose
    // chunks all lie inside the padded row.
    int acc[4] = {0, 0, 0, 0};
    int sxl = 0;
    int i = 0;
    for (; i + D < nst; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            sxl = dot8(xq[j][0], 0x11111111u, dot8(xq[j][1], 0x11111111u, sxl));
            mac_a4(r[j], xq[j], acc);
            const int t = min((i + D + j) * 8 + u, last);
            r[j] = __builtin_nontemporal_load(sbase + t * (kTileBytes / 16) + off);
            xq[j] = xp[min(t * 8 + kg, xlast)];
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < nst) {
            // lanes past the strip's last tile, and chunks past the padded row, count as zero
            const int t = (i + j) * 8 + u;
            const bool in = t <= last && t * 8 + kg <= xlast;
            const v2u xv = in ? xq[j] : v2u{0u, 0u};
            sxl = dot8(xv[0], 0x11111111u, dot8(xv[1], 0x11111111u, sxl));
            mac_a4(r[j], xv, acc);
        }
    }
    const int sx = wave_sum(sxl);
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rr[q] = wave_sum(acc[q]);
    if (lane >= 4) return;
    const int v = (lane == 0 ? rr[0] : lane == 1 ? rr[1] : lane == 2 ? rr[2] : rr[3]) - sx;
    const int row = s * kTileRows + sl * 4 + lane;
    if (row < a.N) {
        if (a.y_i32) a.y_i32[row] = v;
        if (a.y_f32) a.y_f32[row] = (float(v) * a.sa[0]) * a.sw;
    }
}

template <int D, bool MS>
__global__ __launch_bounds__(1024) void gemv_a4_fused_kernel(GemvLaunch a) {
    a4_body<D, true, MS>(a);
}

}  // namespace

namespace {

template <bool FUSED>
hipError_t launch_a4(const GemvLaunch &la, int depth, bool ms, hipStream_t stream) {
    if (la.WK < 1 || la.WK > 16) return hipErrorInvalidValue;
    if (FUSED && (la.RUN < 1 || la.RUN > (ms ? kA4SharedMaxRun : kA4FusedMaxRun)))
        return hipErrorInvalidValue;
    GemvLaunch a = la;
    a.KQ = a.KT / a.SG;
    a.KR = a.KT % a.SG;
    a.WQ0 = a.KQ / a.WK;
    a.WR0 = a.KQ % a.WK;
    a.WQ1 = (a.KQ + 1) / a.WK;
    a.WR1 = (a.KQ + 1) % a.WK;
    void *args[] = {&a};
    const void *fn;
#define W2A8_A4(DD)                                                                        \
    fn = !FUSED ? reinterpret_cast<const void *>(&gemv_a4_kernel<DD>)                      \
         : ms   ? reinterpret_cast<const void *>(&gemv_a4_fused_kernel<DD, true>)          \
                : reinterpret_cast<const void *>(&gemv_a4_fused_kernel<DD, false>)
    switch (depth) {
    case 2: W2A8_A4(2); break;
    case 4: W2A8_A4(4); break;
    case 6: W2A8_A4(6); break;
    case 8: W2A8_A4(8); break;
    case 12: W2A8_A4(12); break;
    default: return hipErrorInvalidValue;
    }
#undef W2A8_A4
    const size_t lds = !FUSED ? 0 : ms ? size_t(a.RUN) * 64 : size_t(a.WK) * a.RUN * 64;
    const unsigned gx = unsigned(ms ? (a.NS + a.WK - 1) / a.WK : a.NS);
    return hipLaunchKernel(fn, dim3(gx, unsigned(a.SG)), dim3(unsigned(64 * a.WK)), args, lds,
                           stream);
}

}  // namespace

hipError_t launch_gemv_a4(const GemvLaunch &a, int depth, hipStream_t stream) {
    return launch_a4<false>(a, depth, false, stream);
}

hipError_t launch_gemv_a4_fused(const GemvLaunch &a, int depth, bool shared, hipStream_t stream) {
    return launch_a4<true>(a, depth, shared, stream);
}

hipError_t launch_gemv_a4_slice(const GemvLaunch &la, int depth, hipStream_t stream) {
    if (int64_t(la.NS) * 8 > INT32_MAX) return hipErrorInvalidValue;
    GemvLaunch a = la;
    void *args[] = {&a};
    const void *fn;
    switch (depth) {
    case 2: fn = reinterpret_cast<const void *>(&gemv_a4_slice_kernel<2>); break;
    case 4: fn = reinterpret_cast<const void *>(&gemv_a4_slice_kernel<4>); break;
    case 6: fn = reinterpret_cast<const void *>(&gemv_a4_slice_kernel<6>); break;
    case 8: fn = reinterpret_cast<const void *>(&gemv_a4_slice_kernel<8>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(unsigned(a.NS) * 8), dim3(64), args, 0, stream);
}

}  // namespace w2a8
