// Per-token absmax quantization of bf16 activations to int8 (gfx950).
//
// The pages fix 8-bit activations ("如何编译 BitNet W2A8 CUDA 内核并用 test.py
// 运行 GEMV 加速测试？", introduction) but give no quantizer.  Per row m:
//   a = max|x|;  inv = 127/a;  q = clamp(round_half_even(x*inv), -127, 127);
//   s_a = a/127;  a zero row gives q = 0, s_a = 0.
// Every step is a single correctly rounded fp32 operation (the division is
// IEEE, the product is not contracted, v_rndne_f32 rounds half to even), so
// the result is bit-identical to any IEEE implementation of the same steps.
//
// One 256-thread workgroup per row: a vectorised max pass, a block max, then
// a quantize pass that re-reads the row from L2.
//
// The int4 variant ("a4.8" activations of "微软BitNet：1-bit量化大模型CPU
//部署实践", named there without a formula) takes the same steps with 7 in
// place of 127 and writes the A4I layout (a4.h).
#include "a4.h"
#include "common.h"
#include "device.h"

namespace w2a8 {
namespace {


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
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float red[4];
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    if (amax == 0.0f) {
        for (int k = tid; k < K; k += 256) out[k] = 0;
        if (tid == 0) sa[m] = 0.0f;
        return;
    }
    const float inv = 127.0f / amax;
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
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float red[4];
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// q = clamp(round_half_even(x * inv), -7, 7) as a two's complement nibble.
__device__ __forceinline__ uint32_t q4(float x, float inv) {
    float r = __builtin_rintf(x * inv);
    r = fminf(fmaxf(r, -7.0f), 7.0f);
    return uint32_t(int(r)) & 15u;
}

// Two 32-bit words of one 16-value chunk in the A4I layout: byte j of the
// first word holds values j (low nibble) and 8 + j (high), byte j of the
// second word values 4 + j and 12 + j.
__device__ __forceinline__ void chunk_a4(const float (&v)[16], float inv, uint32_t &w0,
                                         uint32_t &w1) {
    w0 = w1 = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w0 |= (q4(v[j], inv) | (q4(v[8 + j], inv) << 4)) << (8 * j);
        w1 |= (q4(v[4 + j], inv) | (q4(v[12 + j], inv) << 4)) << (8 * j);
    }
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
    const float inv = amax == 0.0f ? 0.0f : 7.0f / amax;
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

}  // namespace

hipError_t launch_quant_a4(const uint16_t *xb, int M, int K, uint8_t *xq4, float *sa,
                           hipStream_t stream) {
    void *args[] = {const_cast<uint16_t **>(&xb), &M, &K, &xq4, &sa};
    return hipLaunchKernel(reinterpret_cast<const void *>(&quant_a4_kernel), dim3(unsigned(M)),
                           dim3(256), args, 0, stream);
}

hipError_t launch_quant(const uint16_t *xb, int M, int K, int8_t *xq, float *sa,
                        hipStream_t stream) {
    void *args[] = {const_cast<uint16_t **>(&xb), &M, &K, &xq, &sa};
    return hipLaunchKernel(reinterpret_cast<const void *>(&quant_kernel), dim3(unsigned(M)),
                           dim3(256), args, 0, stream);
}

}  // namespace w2a8
