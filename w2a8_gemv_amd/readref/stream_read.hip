// Pure streaming read of a device buffer, for measurement only: the time one
// cold pass over the same bytes takes on this device with no arithmetic, no
// activation traffic and no output (the attainable floor a GEMV over a matrix
// of that size is compared with).  Not part of the W2A8 library.
//
// The buffer is T tiles of 1 KiB (one 16-byte load per lane of a wave64).
// Wave w of G reads the contiguous tiles [w*T/G, (w+1)*T/G) with two batches
// of four non-temporal loads in flight, the same load pattern as the GEMV.
// The loaded words are folded into one value that is stored only if it equals
// a sentinel the caller never passes, so no load is optimised away and
// nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kBatch = 4;

__device__ __forceinline__ void load_batch(const v4u *p, int t, int last, v4u (&w)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) w[u] = __builtin_nontemporal_load(p + min(t + u, last) * 64);
    __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(256) void stream_read_kernel(const v4u *p, int64_t T, int G,
                                                          uint32_t sentinel, uint32_t *out) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * 4 + (int(threadIdx.x) >> 6));
    if (wave >= G) return;
    const int64_t t0 = int64_t(wave) * T / G, t1 = int64_t(wave + 1) * T / G;
    const int n = int(t1 - t0);
    if (n <= 0) return;
    const v4u *q = p + t0 * 64 + lane;
    const int last = n - 1;
    const int nb = (n + kBatch - 1) / kBatch;
    v4u acc = {0u, 0u, 0u, 0u};
    v4u a[kBatch], b[kBatch];
    load_batch(q, 0, last, a);
    load_batch(q, kBatch, last, b);
    int i = 0;
    for (; i + 2 < nb; i += 2) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) acc ^= a[u];
        load_batch(q, (i + 2) * kBatch, last, a);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) acc ^= b[u];
        load_batch(q, (i + 3) * kBatch, last, b);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) acc ^= a[u];
    if (i + 1 < nb) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) acc ^= b[u];
    }
    const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (v == sentinel) out[wave] = v;
}

}  // namespace

// Enqueue one read of `nbytes` (a positive multiple of 1024) at `p` (16-byte
// aligned) with `waves` waves on `stream`; `out` holds `waves` words (written
// only on a sentinel match).  Returns 0, or -1 for bad arguments, or the HIP
// error of the launch.
extern "C" int w2a8_readref_stream(const void *p, int64_t nbytes, int waves, void *out,
                                   void *stream) {
    if (!p || !out || nbytes <= 0 || nbytes % 1024 != 0 || waves < 1 || waves > (1 << 24) ||
        (reinterpret_cast<uintptr_t>(p) & 15) != 0)
        return -1;
    const int64_t T = nbytes / 1024;
    hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v4u *>(p), T, waves,
                       0x9E3779B9u, static_cast<uint32_t *>(out));
    return int(hipGetLastError());
}
