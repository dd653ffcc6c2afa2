// Per-token absmax quantization of bf16 activations to int8 (gfx950).
//
// The pages fix 8-bit activations ("如何编译 BitNet W2A8 CUDA 内核并用 test.py
// 运行 GEMV 加速测试？", introduction) but give no quantizer.  Per row m:
//   a = max|x|;  inv = min(127/a, FLT_MAX);  q = clamp(round_half_even(x*inv), -127, 127);
//   s_a = a/127;  a zero row gives q = 0, s_a = 0.
// Every step is a single correctly rounded fp32 operation (the division is
// IEEE, the product is not contracted, v_rndne_f32 rounds half to even), so
// the result is bit-identical to any IEEE implementation of the same steps.
//
// K a multiple of 8 up to 32768: one workgroup per row, each lane holding
// one to four chunks of 8 values in registers (one read of the row, a row
// maximum across lanes and waves, then quantize and store from the same
// registers).  Other K: one 256-thread workgroup per row, a vectorised max
// pass, a block max, then a quantize pass that re-reads the row from L2.
//
// The int4 variant (the "a4.8" activations that
// "使用 BitNet 框架部署 1-bit LLM：三元权重量化、LUT 矩阵乘加速与 GPU 运行时优化",
// section "GPU 运行时优化与低延迟推理管道", names without a formula) takes the
// same steps with 7 in place of 127 and writes the A4I layout (a4.h).
#include "a4.h"
#include "common.h"
#include "device.h"

namespace w2a8 {
namespace {

// Longest row of the one-read kernels (at most 4 chunks per lane over 1024
// lanes: 32768 values in 8-value chunks; the int4 kernel's 16-value chunks
// and extra slot fit as well).
constexpr int kQuantRowsMaxK = 32768;


__global__ __launch_bounds__(256) void quant_kernel(const uint16_t *xb, int M, int K, int8_t *xq,
                                                    float *sa) {
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t *row = xb + int64_t(m) * K;
    int8_t *out = xq + int64_t(m) * K;
    // Rows are 16-byte aligned (input) and 8-byte aligned (output) when K%8 == 0.
    const bool vec = (K & 7) == 0;

    float amax = 0.0f;
    if (vec) {
        const v4u *r8 = reinterpret_cast<const v4u *>(row);
        for (int c = tid; c < K / 8; c += 256) {
            const v4u v = r8[c];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(v[j])), fabsf(hi_bf16(v[j]))));
        }
    } else {
        for (int k = tid; k < K; k += 256) amax = fmaxf(amax, fabsf(lo_bf16(row[k])));
    }
    amax = wave_max_nonneg(amax);
    __shared__ float red[4];
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    if (amax == 0.0f) {
        for (int k = tid; k < K; k += 256) out[k] = 0;
        if (tid == 0) sa[m] = 0.0f;
        return;
    }
    const float inv = fminf(127.0f / amax, __FLT_MAX__);
    if (vec) {
        const v4u *r8 = reinterpret_cast<const v4u *>(row);
        v2u *o8 = reinterpret_cast<v2u *>(out);
        for (int c = tid; c < K / 8; c += 256) {
            const v4u v = r8[c];
            uint32_t o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t a = v[2 * h], b = v[2 * h + 1];
                o[h] = q8(lo_bf16(a), inv) | (q8(hi_bf16(a), inv) << 8) |
                       (q8(lo_bf16(b), inv) << 16) | (q8(hi_bf16(b), inv) << 24);
            }
            o8[c] = v2u{o[0], o[1]};
        }
    } else {
        for (int k = tid; k < K; k += 256) out[k] = int8_t(q8(lo_bf16(row[k]), inv));
    }
    if (tid == 0) sa[m] = amax / 127.0f;
}

// Row maximum over a workgroup of up to 16 waves, given each lane's
// maximum: within each wave by lane exchanges, then across the waves
// through LDS (each wave writes its maximum, wave 0 zeroes the unused
// entries, and every lane reads all 16 with four 16-byte reads).
__device__ __forceinline__ float block_absmax(float amax, float (&red)[16]) {
    amax = wave_max_nonneg(amax);
    const int tid = int(threadIdx.x);
    const int nw = int(blockDim.x) >> 6;
    if (nw > 1) {
        if ((tid & 63) == 0) red[tid >> 6] = amax;
        if (tid >= nw && tid < 16) red[tid] = 0.0f;
        __syncthreads();
        const v4u *r4 = reinterpret_cast<const v4u *>(red);
        const v4u q0 = r4[0], q1 = r4[1], q2 = r4[2], q3 = r4[3];
        float m4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m4[i] = fmaxf(fmaxf(__uint_as_float(q0[i]), __uint_as_float(q1[i])),
                          fmaxf(__uint_as_float(q2[i]), __uint_as_float(q3[i])));
        amax = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    }
    return amax;
}

// One workgroup per row (K % 8 == 0, K <= 32768), CPL chunks of 8 values per
// lane (chunk tid + i * blockDim): the lanes load the row once, take the
// maximum (block_absmax), and quantize and store the chunks held in
// registers.  Same per-element operations (q8) as quant_kernel.
template <int CPL>
__global__ __launch_bounds__(1024) void quant_rows_kernel(const uint16_t *xb, int M, int K,
                                                          int8_t *xq, float *sa) {
    const int tid = int(threadIdx.x);
    const int bd = int(blockDim.x);
    const int m = int(blockIdx.x);
    const int nc = K >> 3;
    const v4u *r8 = reinterpret_cast<const v4u *>(xb + int64_t(m) * K);
    v2u *o8 = reinterpret_cast<v2u *>(xq + int64_t(m) * K);
    v4u v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        v[i] = tid + i * bd < nc ? r8[tid + i * bd] : v4u{0u, 0u, 0u, 0u};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(v[i][j])), fabsf(hi_bf16(v[i][j]))));
    __shared__ __attribute__((aligned(16))) float red[16];
    amax = block_absmax(amax, red);
    const float inv = amax == 0.0f ? 0.0f : fminf(127.0f / amax, __FLT_MAX__);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = tid + i * bd;
        if (c < nc) {
            uint32_t o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t a = v[i][2 * h], b = v[i][2 * h + 1];
                o[h] = q8(lo_bf16(a), inv) | (q8(hi_bf16(a), inv) << 8) |
                       (q8(lo_bf16(b), inv) << 16) | (q8(hi_bf16(b), inv) << 24);
            }
            o8[c] = v2u{o[0], o[1]};
        }
    }
    if (tid == 0) sa[m] = amax / 127.0f;
}

// Row maximum of |x| over a workgroup of 256 threads.
__device__ __forceinline__ float row_absmax(const uint16_t *row, int K, bool vec) {
    const int tid = threadIdx.x;
    float amax = 0.0f;
    if (vec) {
        const v4u *r8 = reinterpret_cast<const v4u *>(row);
        for (int c = tid; c < K / 8; c += 256) {
            const v4u v = r8[c];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(v[j])), fabsf(hi_bf16(v[j]))));
        }
    } else {
        for (int k = tid; k < K; k += 256) amax = fmaxf(amax, fabsf(lo_bf16(row[k])));
    }
    amax = wave_max_nonneg(amax);
    __shared__ float red[4];
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One 256-thread workgroup per row; each thread writes 32-value granules
// (16 bytes).  Values past K are written as zero nibbles.
__global__ __launch_bounds__(256) void quant_a4_kernel(const uint16_t *xb, int M, int K,
                                                       uint8_t *xq4, float *sa) {
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t *row = xb + int64_t(m) * K;
    const int G = (K + 31) / 32;
    v4u *out = reinterpret_cast<v4u *>(xq4 + int64_t(m) * G * 16);
    const bool vec = (K & 7) == 0;
    const float amax = row_absmax(row, K, vec);
    const float inv = amax == 0.0f ? 0.0f : fminf(7.0f / amax, __FLT_MAX__);
    for (int g = tid; g < G; g += 256) {
        uint32_t w[4];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float v[16];
            const int k0 = 32 * g + 16 * c;
            if (vec && k0 + 16 <= K) {
                const v4u *p = reinterpret_cast<const v4u *>(row + k0);
                const v4u a = p[0], b = p[1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = lo_bf16(a[j]);
                    v[2 * j + 1] = hi_bf16(a[j]);
                    v[8 + 2 * j] = lo_bf16(b[j]);
                    v[8 + 2 * j + 1] = hi_bf16(b[j]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = k0 + i < K ? lo_bf16(row[k0 + i]) : 0.0f;
            }
            chunk_a4(v, inv, w[2 * c], w[2 * c + 1]);
        }
        out[g] = v4u{w[0], w[1], w[2], w[3]};
    }
    if (tid == 0) sa[m] = amax / 7.0f;
}

// K % 16 == 0 and K <= 32768: one workgroup per row, CPL 16-value chunks
// per lane (chunk tid + i * blockDim), as quant_rows_kernel: the row is read
// once, its maximum taken (block_absmax), and each lane quantizes the chunks
// it holds into their 8 bytes of the A4I row.  With an odd number of chunks
// the lane of chunk index nc (one past the last; the launch always provides
// it) writes the zero half of the last granule.  Same per-element operations
// (q4) as quant_a4_kernel.
template <int CPL>
__global__ __launch_bounds__(1024) void quant_a4_rows_kernel(const uint16_t *xb, int M, int K,
                                                             uint8_t *xq4, float *sa) {
    const int tid = int(threadIdx.x);
    const int bd = int(blockDim.x);
    const int m = int(blockIdx.x);
    const int nc = K >> 4;                        // 16-value chunks of the row
    const int G = (K + 31) / 32;                  // 32-value granules (16 bytes each)
    const v4u *r8 = reinterpret_cast<const v4u *>(xb + int64_t(m) * K);
    v2u *o8 = reinterpret_cast<v2u *>(xq4 + int64_t(m) * G * 16);
    v4u a[CPL], b[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = tid + i * bd;
        a[i] = b[i] = v4u{0u, 0u, 0u, 0u};
        if (c < nc) {
            a[i] = r8[2 * c];
            b[i] = r8[2 * c + 1];
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(a[i][j])), fabsf(hi_bf16(a[i][j]))));
            amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(b[i][j])), fabsf(hi_bf16(b[i][j]))));
        }
    __shared__ __attribute__((aligned(16))) float red[16];
    amax = block_absmax(amax, red);
    const float inv = amax == 0.0f ? 0.0f : fminf(7.0f / amax, __FLT_MAX__);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = tid + i * bd;
        if (c < nc) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = lo_bf16(a[i][j]);
                v[2 * j + 1] = hi_bf16(a[i][j]);
                v[8 + 2 * j] = lo_bf16(b[i][j]);
                v[8 + 2 * j + 1] = hi_bf16(b[i][j]);
            }
            uint32_t w0, w1;
            chunk_a4(v, inv, w0, w1);
            o8[c] = v2u{w0, w1};
        } else if (c == nc && (nc & 1)) {
            o8[c] = v2u{0u, 0u};
        }
    }
    if (tid == 0) sa[m] = amax / 7.0f;
}

// Chunks per lane and workgroup size of the one-read kernels: `slots`
// chunk slots over at most 1024 threads (at most 4 per lane), in whole waves.
int rows_cpl(int slots) { return (slots + 1023) / 1024; }
int rows_threads(int slots, int cpl) { return ((slots + cpl - 1) / cpl + 63) / 64 * 64; }

template <typename F>
hipError_t launch_rows(F *const (&fns)[4], int slots, void **args, int M, hipStream_t stream) {
    const int cpl = rows_cpl(slots);
    return hipLaunchKernel(reinterpret_cast<const void *>(fns[cpl - 1]), dim3(unsigned(M)),
                           dim3(unsigned(rows_threads(slots, cpl))), args, 0, stream);
}

}  // namespace

// K % 16 == 0 and K <= 32768: one workgroup per row over the chunks and the
// one slot past them (K/16 + 1 slots), 1 to 4 16-value chunks per lane
// (quant_a4_rows_kernel).  Other K: one 256-thread workgroup per row, two
// passes (quant_a4_kernel).
hipError_t launch_quant_a4(const uint16_t *xb, int M, int K, uint8_t *xq4, float *sa,
                           hipStream_t stream) {
    void *args[] = {const_cast<uint16_t **>(&xb), &M, &K, &xq4, &sa};
    if ((K & 15) == 0 && K <= kQuantRowsMaxK) {
        using Fn = void(const uint16_t *, int, int, uint8_t *, float *);
        static Fn *const fns[4] = {&quant_a4_rows_kernel<1>, &quant_a4_rows_kernel<2>,
                                   &quant_a4_rows_kernel<3>, &quant_a4_rows_kernel<4>};
        return launch_rows(fns, K / 16 + 1, args, M, stream);
    }
    return hipLaunchKernel(reinterpret_cast<const void *>(&quant_a4_kernel), dim3(unsigned(M)),
                           dim3(256), args, 0, stream);
}

// K % 8 == 0 and K <= 32768: one workgroup per row, 1 to 4 chunks of 8
// values per lane (quant_rows_kernel).  Other K: one 256-thread workgroup
// per row, two passes (quant_kernel).
hipError_t launch_quant(const uint16_t *xb, int M, int K, int8_t *xq, float *sa,
                        hipStream_t stream) {
    void *args[] = {const_cast<uint16_t **>(&xb), &M, &K, &xq, &sa};
    if ((K & 7) == 0 && K <= kQuantRowsMaxK) {
        using Fn = void(const uint16_t *, int, int, int8_t *, float *);
        static Fn *const fns[4] = {&quant_rows_kernel<1>, &quant_rows_kernel<2>,
                                   &quant_rows_kernel<3>, &quant_rows_kernel<4>};
        return launch_rows(fns, K / 8, args, M, stream);
    }
    return hipLaunchKernel(reinterpret_cast<const void *>(&quant_kernel), dim3(unsigned(M)),
                           dim3(256), args, 0, stream);
}

}  // namespace w2a8
