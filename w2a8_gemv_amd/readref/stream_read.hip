// Plain streaming reads of a device buffer, for measurement only (not part of
// the W2A8 library): what one cold pass over N bytes costs on this device with
// no arithmetic and no output, under a range of load shapes, so that a GEMV
// over a matrix of that size can be compared with the best plain read of the
// same bytes.
//
// The buffer is read in chunks of 64*W bytes: one load instruction of a wave64
// with W bytes per lane (W = 4, 8 or 16: global_load_dword / _dwordx2 /
// _dwordx4).  G waves share the chunks, either as contiguous runs (wave w
// reads chunks [w*C/G, (w+1)*C/G)) or strided (wave w reads chunks w, w+G,
// w+2G, ...).  Each wave keeps a ring of D loads in flight: after the first D
// loads it waits for the oldest one, folds it into a running value and issues
// the next load into the freed slot, so D-1 loads stay outstanding throughout
// (loads return in order, so the compiler's wait counts are exact).  Past the
// end of its run a wave re-issues its last chunk (an address it owns) rather
// than branching, and ignores the value.  Loads are non-temporal or plain.
//
// The folded value is stored only if it equals a sentinel the caller never
// passes, so no load is optimised away and nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

template <int W> struct Vec;
template <> struct Vec<4> { typedef uint32_t T; };
template <> struct Vec<8> { typedef v2u T; };
template <> struct Vec<16> { typedef v4u T; };

__device__ __forceinline__ uint32_t fold(uint32_t v) { return v; }
__device__ __forceinline__ uint32_t fold(v2u v) { return v[0] ^ v[1]; }
__device__ __forceinline__ uint32_t fold(v4u v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

template <int W, bool NT>
__device__ __forceinline__ typename Vec<W>::T ld(const typename Vec<W>::T *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int W, int D, bool NT, bool STRIDED>
__global__ __launch_bounds__(256) void read_kernel(const uint8_t *buf, int64_t nchunks, int G,
                                                   uint32_t sentinel, uint32_t *out) {
    typedef typename Vec<W>::T T;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * 4 + (int(threadIdx.x) >> 6));
    if (wave >= G) return;
    int64_t first, step, n;
    if constexpr (STRIDED) {
        first = wave;
        step = G;
        n = wave < nchunks ? (nchunks - 1 - wave) / G + 1 : 0;
    } else {
        first = int64_t(wave) * nchunks / G;
        step = 1;
        n = (int64_t(wave) + 1) * nchunks / G - first;
    }
    if (n <= 0) return;
    const T *base = reinterpret_cast<const T *>(buf) + lane;
    // Running address of the next chunk to load, clamped to the wave's last
    // chunk (an address it owns) once the run is exhausted.
    const int64_t inc = step * 64;
    const T *last = base + (first + (n - 1) * step) * 64;
    const T *addr = base + first * 64;
    T r[D];
    // Keep the program order (fill slots 0..D-1; then consume slot j and
    // reload it): the scheduler would otherwise regroup the loads, and the
    // wait at the loop head would cover several of them.
#pragma unroll
    for (int j = 0; j < D; ++j) {
        r[j] = ld<W, NT>(addr < last ? addr : last);
        addr += inc;
        __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t acc = 0;
    int64_t i = 0;   // chunks consumed
    for (; i + D < n; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            acc ^= fold(r[j]);
            r[j] = ld<W, NT>(addr < last ? addr : last);
            addr += inc;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j)
        if (i + j < n) acc ^= fold(r[j]);
    if (acc == sentinel) out[wave] = acc;
}

__global__ __launch_bounds__(256) void empty_kernel(int G, uint32_t sentinel, uint32_t *out) {
    const int wave = int(blockIdx.x) * 4 + (int(threadIdx.x) >> 6);
    if (wave < G && uint32_t(wave) == sentinel) out[wave] = 1;
}

typedef void (*ReadFn)(const uint8_t *, int64_t, int, uint32_t, uint32_t *);

template <int W, bool NT, bool S>
ReadFn pick_depth(int d) {
    switch (d) {
    case 2: return read_kernel<W, 2, NT, S>;
    case 4: return read_kernel<W, 4, NT, S>;
    case 8: return read_kernel<W, 8, NT, S>;
    case 12: return read_kernel<W, 12, NT, S>;
    case 16: return read_kernel<W, 16, NT, S>;
    default: return nullptr;
    }
}

template <int W>
ReadFn pick(int d, bool nt, bool strided) {
    if (nt) return strided ? pick_depth<W, true, true>(d) : pick_depth<W, true, false>(d);
    return strided ? pick_depth<W, false, true>(d) : pick_depth<W, false, false>(d);
}

constexpr uint32_t kSentinel = 0x9E3779B9u;

}  // namespace

// Enqueue one read of `nbytes` at `p` on `stream` with `waves` waves
// (workgroups of 4 waves): loads of `width` bytes per lane (4, 8 or 16),
// `depth` loads in flight per wave (2, 4, 8, 12 or 16), non-temporal when
// `nt`, strided chunk assignment when `strided`.  `nbytes` must be a positive
// multiple of 64*width and `p` aligned to `width`; `out` holds `waves` words
// (written only on a sentinel match).  Returns 0, -1 for bad arguments, or the
// HIP error of the launch.
extern "C" int w2a8_readref_read(const void *p, int64_t nbytes, int waves, int width, int depth,
                                 int nt, int strided, void *out, void *stream) {
    if (!p || !out || nbytes <= 0 || waves < 1 || waves > (1 << 24)) return -1;
    if (!(width == 4 || width == 8 || width == 16)) return -1;
    if (nbytes % (64 * width) != 0 || (reinterpret_cast<uintptr_t>(p) & (width - 1)) != 0)
        return -1;
    ReadFn fn = width == 4 ? pick<4>(depth, nt != 0, strided != 0)
              : width == 8 ? pick<8>(depth, nt != 0, strided != 0)
                           : pick<16>(depth, nt != 0, strided != 0);
    if (!fn) return -1;
    hipLaunchKernelGGL(fn, dim3(unsigned((waves + 3) / 4)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(p),
                       nbytes / (64 * width), waves, kSentinel, static_cast<uint32_t *>(out));
    return int(hipGetLastError());
}

// Enqueue a kernel of `waves` waves that reads nothing: the launch and
// dispatch cost alone, for comparison.
extern "C" int w2a8_readref_empty(int waves, void *out, void *stream) {
    if (!out || waves < 1 || waves > (1 << 24)) return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), waves, kSentinel,
                       static_cast<uint32_t *>(out));
    return int(hipGetLastError());
}
