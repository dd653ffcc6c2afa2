// Fused W2A8 linear layer for one token on the ring weight stream: bf16 row
// -> per-token absmax int8 codes -> exact integer product with the ternary
// weights -> fp32 output, in one launch.
//
// What it computes: the quantizer of the a3 step (8-bit activations of
// "如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？", introduction;
// per-token absmax with 127 levels per side), the integer product of its
// sections "运行 test.py 做 GEMV 基准测试" / "如何判断结果", and the scale
// epilogue of "Windows 上跑通 BitNet b1.58：…部署实录" §3.1.  Every element goes
// through the quantizer kernel's correctly rounded fp32 steps (q8,
// common.h), so codes, scale and outputs are bit-identical to
// quant_act_int8 followed by w2a8_gemv.
//
// The weight stream, decode and reductions are those of the ring GEMV
// (gemv_ring.hip): each wave keeps a ring of D tiles in flight.  What this
// kernel adds, before the stream:
//  * each thread loads the first pieces of its share of the row (for the
//    maximum) and the first chunk it will quantize, before the weight ring,
//    so those L2 hits do not wait behind the weights in the in-order load
//    counter;
//  * after the ring is issued: the rest of the maximum share, DPP within
//    waves, one barrier across them, inv = min(127/amax, FLT_MAX) and
//    sa = amax/127;
//  * quantization into LDS, 16 values (one 16-byte chunk) per step, values
//    past K as zeros (so any K works: the pad codes meet zero activations);
//  * the stream then reads each tile's chunk from LDS.
// Work split (shared k-ranges): a workgroup of WK waves takes WK consecutive
// strips over one k-range (one wave each) and quantizes the k-range once
// into one LDS region that all its waves read, so the row's maximum and
// quantization are shared by WK strips.  (Per-wave runs, each wave
// quantizing its own run as the W2A4 kernel does for plans with several
// waves per strip, measured slower here than the workgroup kernel's fused
// variant: 5.62 against 5.22 us at 13824 x 2560.)
#include "a4.h"
#include "device.h"
#include "linear_ring.h"

namespace w2a8 {
namespace {

struct RingAcc8 {
    int a1[4], a4[4], a16[4];
};

// One lane slot of a tile: 4 rows x 16 k of codes c = w + 1 against 16
// activation bytes; masks leave c, 4c, 16c, 16c in the bytes, and the three
// accumulators (scales 1, 4, 16) are divided back exactly at the end.
__device__ __forceinline__ void mac8(const v4u w, const v4u xv, RingAcc8 &acc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = w[q];
        acc.a1[q] = dot4(v & 0x03030303u, xv[0], acc.a1[q]);
        acc.a4[q] = dot4(v & 0x0C0C0C0Cu, xv[1], acc.a4[q]);
        acc.a16[q] = dot4(v & 0x30303030u, xv[2], acc.a16[q]);
        acc.a16[q] = dot4((v >> 2) & 0x30303030u, xv[3], acc.a16[q]);
    }
}

__device__ __forceinline__ int sum16(const v4u x, int s) {
    s = dot4(x[0], 0x01010101u, s);
    s = dot4(x[1], 0x01010101u, s);
    s = dot4(x[2], 0x01010101u, s);
    return dot4(x[3], 0x01010101u, s);
}

__device__ __forceinline__ float absmax8(float m, const v4u v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(lo_bf16(v[i])), fabsf(hi_bf16(v[i]))));
    return m;
}

// 16 bf16 values (two 16-byte pieces) -> 16 int8 codes, value 4q + j in byte
// j of word q.
__device__ __forceinline__ v4u codes16(const v4u lo, const v4u hi, float inv) {
    v4u o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t p = q < 2 ? lo[2 * q] : hi[2 * q - 4];
        const uint32_t r = q < 2 ? lo[2 * q + 1] : hi[2 * q - 3];
        o[q] = q8(lo_bf16(p), inv) | (q8(hi_bf16(p), inv) << 8) | (q8(lo_bf16(r), inv) << 16) |
               (q8(hi_bf16(r), inv) << 24);
    }
    return o;
}

template <int D>
__global__ __launch_bounds__(1024) void linear_ring_kernel(GemvLaunch a) {
    __shared__ __attribute__((aligned(16))) float wmax[16];
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Strip s (past the last strip: loads from the last strip, no output).
    const int s = int(blockIdx.x) * a.WK + wv;
    const bool live = s < a.NS;
    const int g = int(blockIdx.y);
    const bool big = g < a.KR;
    // The k-range: tiles w0 .. w0+n-1; loads past it re-read its last tile.
    const int w0 = g * a.KQ + min(g, a.KR);
    const int n = a.KQ + (big ? 1 : 0);
    const int kg = lane & 7, rg = lane >> 3;
    const int last = min(max(w0, w0 + n - 1), a.KT - 1);
    const v4u *sbase =
        reinterpret_cast<const v4u *>(a.wp + int64_t(min(s, a.NS - 1)) * a.KT * kTileWords);
    const int K = a.K;
    const int bd = int(blockDim.x);
    const v4u *r8 = reinterpret_cast<const v4u *>(a.xb);

    // 0. The first share of the row maximum and the first chunk to quantize
    //    (chunk c of the k-range holds values 16(8 w0 + c) .. +15).
    const int qfirst = tid, qstride = bd;
    v4u mx0 = {0u, 0u, 0u, 0u}, mx1 = mx0, qa = mx0, qb = mx0;
    if (tid < (K >> 3)) mx0 = r8[tid];
    if (tid + bd < (K >> 3)) mx1 = r8[tid + bd];
    const bool qpre = qfirst < 8 * n && 16 * (8 * w0 + qfirst) + 16 <= K;
    if (qpre) {
        const v4u *p = reinterpret_cast<const v4u *>(a.xb + 16 * (8 * w0 + qfirst));
        qa = p[0];
        qb = p[1];
    }
    __builtin_amdgcn_sched_barrier(0);

    // 1. Fill the ring: tiles w0 .. w0+D-1 (clamped to `last`).
    v4u r[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        r[j] = __builtin_nontemporal_load(sbase + min(w0 + j, last) * (kTileBytes / 16) + lane);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 2. Row maximum over the workgroup (a zero piece adds nothing).
    float amax = absmax8(absmax8(0.0f, mx0), mx1);
    {
        int c = tid + 2 * bd;
        for (; c + 3 * bd < (K >> 3); c += 4 * bd) {   // four loads in flight
            const v4u v0 = r8[c], v1 = r8[c + bd], v2 = r8[c + 2 * bd], v3 = r8[c + 3 * bd];
            amax = absmax8(absmax8(absmax8(absmax8(amax, v0), v1), v2), v3);
        }
        for (; c < (K >> 3); c += bd) amax = absmax8(amax, r8[c]);
    }
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
    const float inv = amax == 0.0f ? 0.0f : fminf(127.0f / amax, __FLT_MAX__);
    const float sa = amax / 127.0f;

    // 3. Quantize the k-range into LDS.
    v4u *xl = reinterpret_cast<v4u *>(smem);
    for (int c = qfirst; c < 8 * n; c += qstride) {
        const int k0 = 16 * (8 * w0 + c);
        v4u o;
        if (k0 + 16 <= K) {
            v4u lo = qa, hi = qb;
            if (!(qpre && c == qfirst)) {
                const v4u *p = reinterpret_cast<const v4u *>(a.xb + k0);
                lo = p[0];
                hi = p[1];
            }
            o = codes16(lo, hi, inv);
        } else {
            o = v4u{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (k0 + i < K)
                    o[i >> 2] |= q8(__uint_as_float(uint32_t(a.xb[k0 + i]) << 16), inv)
                                 << (8 * (i & 3));
        }
        xl[c] = o;
    }
    __syncthreads();

    // 4. Stream: consume tile i of the run, reload its slot with tile i + D.
    const int ns = live ? n : 0;
    RingAcc8 acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc.a1[q] = acc.a4[q] = acc.a16[q] = 0;
    int sxl = 0;
    int i = 0;
    for (; i + D < ns; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const v4u xv = xl[(i + j) * 8 + kg];
            sxl = sum16(xv, sxl);
            mac8(r[j], xv, acc);
            r[j] = __builtin_nontemporal_load(sbase + min(w0 + i + D + j, last) * (kTileBytes / 16) +
                                              lane);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
        if (i + j < ns) {
            const v4u xv = xl[(i + j) * 8 + kg];
            sxl = sum16(xv, sxl);
            mac8(r[j], xv, acc);
        }
    }
    const int sx = sum8(sxl);

    // 5. Reduce over the 8 lanes of a row group (sum_k w*x = sum_k c*x -
    //    sum_k x); lane 8 rg + q (q < 4) owns row 4 rg + q of the strip.
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rr[q] = sum8(acc.a1[q] + (acc.a4[q] >> 2) + (acc.a16[q] >> 4));
    const int tot = (kg == 0 ? rr[0] : kg == 1 ? rr[1] : kg == 2 ? rr[2] : rr[3]) - sx;
    const bool owner = live && kg < 4;
    const int row = s * kTileRows + rg * 4 + kg;
    int v = tot;
    if (a.SG > 1 && !(owner && split_add(a.ws_row + row, n, tot, a.KT, &v))) return;
    if (owner && row < a.N) {
        if (a.y_i32) a.y_i32[row] = v;
        a.y_f32[row] = (float(v) * sa) * a.sw;
    }
}

int64_t cdiv(int64_t x, int64_t y) { return (x + y - 1) / y; }

}  // namespace

bool fused_ring_plan(GemvLaunch *a, int max_run, int max_shared_run) {
    const int64_t NS = a->NS, KT = a->KT;
    if (a->WK == 1) {
        int64_t SG = a->SG;
        const bool fill8 = cdiv(NS, 8) * 8 - NS <= NS / 32;
        const int64_t WS = std::min<int64_t>(NS, fill8 && (SG > 1 || NS >= 1536) ? 8 : 4);
        if (SG > 1 && cdiv(NS, WS) * SG < 200) SG = std::min(KT, 2 * SG);
        if (cdiv(KT, SG) > max_shared_run) SG = cdiv(KT, max_shared_run);
        a->SG = int(SG);
        a->WK = int(WS);
        a->RUN = int(cdiv(KT, SG));
        return true;
    }
    if (a->RUN <= max_run) return false;
    int64_t SG = a->SG;
    int64_t ktw = cdiv(KT, SG);
    if (ktw > 16 * int64_t(max_run)) {
        SG = cdiv(KT, 16 * int64_t(max_run));
        ktw = cdiv(KT, SG);
    }
    const int64_t WK = std::min<int64_t>(16, std::max<int64_t>(a->WK, cdiv(ktw, max_run)));
    a->SG = int(SG);
    a->WK = int(WK);
    a->RUN = int(cdiv(ktw, WK));
    return false;
}

LinearKernel linear_layer_plan(const GemvPolicy &pol, int64_t NS, int64_t KT, int cus, bool int4,
                               GemvLaunch *a, int *depth) {
    a->NS = int(NS);
    a->KT = int(KT);
    *depth = 4;
    gemv_ring_plan(pol, NS, KT, cus, &a->WK, &a->SG, &a->RUN, depth);
    a->unroll = *depth;
    // Shared k-ranges of fewer than 12 tiles keep depth 4 whatever the ring
    // GEMV's plan: depth 8 there measured slower (int8, us: 3200 x 10240,
    // runs of 8: 5.87 against 5.58; 2560 x 27648, runs of 9: 8.10 against
    // 7.43; int4 7.48 against 7.23).
    if (int4) {
        if (!fused_ring_plan(a, kA4FusedMaxRun, kA4SharedMaxRun)) return kLinearPerWave;
        if (a->RUN < 12) *depth = 4;
        a->unroll = *depth;
        return kLinearShared;
    }
    // One wave per strip: shared k-ranges (always the shared plan then).
    // Otherwise the workgroup kernel, which measured faster than the ring
    // with per-wave runs on those plans.
    if (a->WK == 1) {
        fused_ring_plan(a, 0, kLinearSharedMaxRun);
        if (a->RUN < 12) *depth = 4;
        a->unroll = *depth;
        return kLinearShared;
    }
    gemv_plan(pol, NS, KT, cus, &a->WK, &a->SG, &a->RUN, &a->unroll);
    return kLinearWorkgroup;
}

hipError_t launch_linear_ring(const GemvLaunch &la, int depth, hipStream_t stream) {
    if (la.WK < 1 || la.WK > 16 || la.RUN < 1 || la.RUN > kLinearSharedMaxRun ||
        la.RUN < (la.KT + la.SG - 1) / la.SG)
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
#define W2A8_LR(DD) fn = reinterpret_cast<const void *>(&linear_ring_kernel<DD>)
    switch (depth) {
    case 2: W2A8_LR(2); break;
    case 4: W2A8_LR(4); break;
    case 6: W2A8_LR(6); break;
    case 8: W2A8_LR(8); break;
    case 12: W2A8_LR(12); break;
    default: return hipErrorInvalidValue;
    }
#undef W2A8_LR
    const size_t lds = size_t(a.RUN) * kTileK;
    const unsigned gx = unsigned((a.NS + a.WK - 1) / a.WK);
    return hipLaunchKernel(fn, dim3(gx, unsigned(a.SG)), dim3(unsigned(64 * a.WK)), args, lds,
                           stream);
}

}  // namespace w2a8
