// C ABI of the W2A4 variant (int4 activations, A4I layout): size query, host
// packer, quantizer and GEMV.  Validation happens on the host before any HIP
// call, as for the W2A8 entry points.
#include <algorithm>

#include "a4.h"
#include "linear_ring.h"

namespace w2a8 {
namespace {

bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool shape_ok(int64_t N, int64_t K) {
    return N >= 1 && N <= kMaxN && K >= 1 && K <= W2A8_MAX_K;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace
}  // namespace w2a8

using namespace w2a8;

extern "C" {

int64_t w2a4_act_bytes(int64_t M, int64_t K) {
    if (M < 1 || M > kMaxM || K < 1 || K > W2A8_MAX_K) return -1;
    return M * a4_row_bytes(K);
}

int pack_act_int4(const int8_t *q, int64_t M, int64_t K, uint8_t *out, int64_t out_bytes) {
    if (!q || !out) return W2A8_ERR_NULL;
    const int64_t need = w2a4_act_bytes(M, K);
    if (need < 0) return W2A8_ERR_SHAPE;
    if (out_bytes < need) return W2A8_ERR_BUFSIZE;
    const int64_t rb = a4_row_bytes(K);
    for (int64_t m = 0; m < M; ++m) {
        uint8_t *row = out + m * rb;
        for (int64_t b = 0; b < rb; ++b) row[b] = 0;
        const int8_t *src = q + m * K;
        for (int64_t c = 0; c * 16 < K; ++c) {
            for (int i = 0; i < 16 && c * 16 + i < K; ++i) {
                const int v = src[c * 16 + i];
                if (v < -8 || v > 7) return W2A8_ERR_VALUE;
                const int h = i / 4, j = i % 4;
                row[c * 8 + 4 * (h % 2) + j] |= uint8_t((unsigned(v) & 15u) << (4 * (h / 2)));
            }
        }
    }
    return W2A8_OK;
}

int quant_act_int4(const uint16_t *x_bf16, int64_t M, int64_t K, uint8_t *x_q4, float *s_a,
                   void *stream) {
    if (!x_bf16 || !x_q4 || !s_a) return W2A8_ERR_NULL;
    if (M < 1 || M > kMaxM || K < 1 || K > W2A8_MAX_K) return W2A8_ERR_SHAPE;
    if (!aligned_to(x_bf16, 16) || !aligned_to(x_q4, 16) || !aligned_to(s_a, 4))
        return W2A8_ERR_ALIGN;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;
    hipError_t e = launch_quant_a4(x_bf16, int(M), int(K), x_q4, s_a,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

int w2a4_gemv(const void *w_packed, const uint8_t *x_q4, int64_t N, int64_t K, int32_t *y_i32,
              const float *s_a, float s_w, float *y_f32, void *workspace, int64_t ws_bytes,
              void *stream) {
    if (!w_packed || !x_q4) return W2A8_ERR_NULL;
    if (!y_i32 && !y_f32) return W2A8_ERR_NULL;
    if (y_f32 && !s_a) return W2A8_ERR_NULL;
    if (!shape_ok(N, K)) return W2A8_ERR_SHAPE;
    const GemvPolicy pol = gemv_policy();
    const bool need_ws = gemv_may_split((K + kTileK - 1) / kTileK, pol);
    if (need_ws && !workspace) return W2A8_ERR_NULL;
    if (!aligned_to(w_packed, 16) || !aligned_to(x_q4, 16) || (y_i32 && !aligned_to(y_i32, 16)) ||
        (y_f32 && !aligned_to(y_f32, 16)) || (s_a && !aligned_to(s_a, 4)) ||
        (need_ws && !aligned_to(workspace, 16)))
        return W2A8_ERR_ALIGN;
    if (need_ws && ws_bytes < 8 * ((N + kTileRows - 1) / kTileRows * kTileRows))
        return W2A8_ERR_BUFSIZE;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;

    const int64_t Np = (N + kTileRows - 1) / kTileRows * kTileRows;
    GemvLaunch a;
    a.wp = static_cast<const uint32_t *>(w_packed);
    a.x = reinterpret_cast<const int8_t *>(x_q4);
    a.xb = nullptr;
    a.M = 1;
    a.y_i32 = y_i32;
    a.y_f32 = y_f32;
    a.sa = s_a;
    a.sw = s_w;
    a.ws_row = static_cast<uint64_t *>(workspace);
    a.N = int(N);
    a.K = int(K);
    a.KT = int((K + kTileK - 1) / kTileK);
    a.NS = int(Np / kTileRows);
    // The int8 GEMV's kernel choice: the row-slice form on matrices of few,
    // short strips, else the ring kernel's plan.
    int depth = 4;
    hipError_t e;
    if (gemv_slice_plan(a.NS, a.KT, dev.cus, &depth)) {
        a.WK = a.SG = 1;
        a.RUN = a.KT;
        a.unroll = depth;
        e = launch_gemv_a4_slice(a, depth, static_cast<hipStream_t>(stream));
    } else {
        gemv_ring_plan(pol, a.NS, a.KT, dev.cus, &a.WK, &a.SG, &a.RUN, &depth);
        a.unroll = depth;
        e = launch_gemv_a4(a, depth, static_cast<hipStream_t>(stream));
    }
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

int w2a4_linear_gemv(const void *w_packed, const uint16_t *x_bf16, int64_t N, int64_t K,
                     float s_w, float *y_f32, int32_t *y_i32, void *workspace, int64_t ws_bytes,
                     void *stream) {
    if (!w_packed || !x_bf16 || !y_f32) return W2A8_ERR_NULL;
    if (!shape_ok(N, K)) return W2A8_ERR_SHAPE;
    const GemvPolicy pol = gemv_policy();
    const bool need_ws = gemv_may_split((K + kTileK - 1) / kTileK, pol);
    if (need_ws && !workspace) return W2A8_ERR_NULL;
    if (!aligned_to(w_packed, 16) || !aligned_to(x_bf16, 16) || !aligned_to(y_f32, 16) ||
        (y_i32 && !aligned_to(y_i32, 16)) || (need_ws && !aligned_to(workspace, 16)))
        return W2A8_ERR_ALIGN;
    if (need_ws && ws_bytes < 8 * ((N + kTileRows - 1) / kTileRows * kTileRows))
        return W2A8_ERR_BUFSIZE;
    DeviceInfo dev;
    int st = current_device(&dev);
    if (st != W2A8_OK) return st;

    const int64_t Np = (N + kTileRows - 1) / kTileRows * kTileRows;
    GemvLaunch a;
    a.wp = static_cast<const uint32_t *>(w_packed);
    a.x = nullptr;
    a.xb = x_bf16;
    a.M = 1;
    a.y_i32 = y_i32;
    a.y_f32 = y_f32;
    a.sa = nullptr;
    a.sw = s_w;
    a.ws_row = static_cast<uint64_t *>(workspace);
    a.N = int(N);
    a.K = int(K);
    a.KT = int((K + kTileK - 1) / kTileK);
    a.NS = int(Np / kTileRows);
    int depth = 4;
    const bool shared = linear_layer_plan(pol, a.NS, a.KT, dev.cus, true, &a, &depth) == kLinearShared;
    hipError_t e = launch_gemv_a4_fused(a, depth, shared, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? W2A8_OK : W2A8_ERR_LAUNCH;
}

}  // extern "C"
