/*
 * w2a8.h — C ABI of libw2a8.so, the MI355X (gfx950) W2A8 linear layer.
 *
 * The layer: ternary weights {-1, 0, 1} packed at 2 bits each, int8
 * activations, exact int32 accumulation, and an fp32 scale epilogue.
 *
 * Sources (cited by page title and section):
 *   [WIN]  "Windows 上跑通 BitNet b1.58：Flash Attention 与 CUDA sm_86 部署实录",
 *          §3.1 "BitLinear 层的三元权重逻辑".
 *   [CPU]  "微软BitNet：1-bit量化大模型CPU部署实践",
 *          §2.1 "1.58-bit量化原理", §2.2 "CPU优化设计", §6.3 "模型微调".
 *   [DEPLOY] "使用 BitNet 框架部署 1-bit LLM：三元权重量化、LUT 矩阵乘加速与
 *          GPU 运行时优化", section "GPU 运行时优化与低延迟推理管道".
 *   [TEST] "如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？",
 *          sections "编译 W2A8 CUDA 内核", "运行 test.py 做 GEMV 基准测试",
 *          "如何判断结果", "限制与注意事项".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Return value: an int status, W2A8_OK (0) on success, otherwise one of
 *   the W2A8_ERR_* codes below.  The library never prints and never aborts.
 *   Arguments are validated on the host before any device work is enqueued;
 *   on an error nothing is enqueued and no output is written (host
 *   functions may have written part of their output when they return
 *   W2A8_ERR_VALUE, see each function).
 * - Ownership: every buffer is owned by the caller.  The library never
 *   allocates, frees or synchronises device memory.  Device pointers are
 *   plain device addresses (e.g. a torch tensor's data_ptr()).
 * - Streams: `stream` is a hipStream_t passed as void*; NULL means the
 *   legacy default stream.  Device entry points only enqueue work on that
 *   stream and return; results are ready when the stream reaches them.
 *   They may be recorded into a HIP graph (they enqueue kernels only, no
 *   memset or copy).
 * - Device: the current HIP device must be a gfx950 GPU (W2A8_ERR_ARCH
 *   otherwise; W2A8_ERR_NODEVICE if there is none).  The library makes no
 *   HIP call when it is loaded; the first device call queries the device.
 * - Layouts: x is [M][K] row-major int8, y is [M][N] row-major.  N, K, M are
 *   element counts (>= 1).  Device pointers to x, y and packed weights must
 *   be 16-byte aligned (W2A8_ERR_ALIGN), scale pointers 4-byte aligned.
 * - Thread safety: every entry point may be called from several host
 *   threads at once.  The library's mutable state is a per-device property
 *   cache and the measurement knobs of w2a8_tuning.h; both are guarded by a
 *   lock (the batched-product kernel choice is one atomic word), and each
 *   call plans its launch from one consistent copy of the knobs, taken when
 *   the call starts.  Two calls in flight at once must not share a
 *   workspace.
 */
#ifndef W2A8_H
#define W2A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum w2a8_status {
    W2A8_OK = 0,
    W2A8_ERR_NULL = 1,      /* a required pointer is NULL                     */
    W2A8_ERR_SHAPE = 2,     /* M, N or K < 1, or above the documented limits  */
    W2A8_ERR_ALIGN = 3,     /* a pointer is not aligned as required           */
    W2A8_ERR_VALUE = 4,     /* a weight outside {-1,0,1}, a code 11, or a
                               tuning knob / forced plan out of range       */
    W2A8_ERR_BUFSIZE = 5,   /* a packed or workspace buffer is too small      */
    W2A8_ERR_NODEVICE = 6,  /* no HIP device / device query failed            */
    W2A8_ERR_ARCH = 7,      /* the current device is not gfx950               */
    W2A8_ERR_LAUNCH = 8,    /* the kernel launch was rejected by the runtime  */
    W2A8_ERR_SCRATCH = 9    /* w2a8_gemv_noalloc: shape beyond its scratch    */
};

/* Version of the packed weight layout below; stored packed weights are only
 * valid for the same version. */
#define W2A8_LAYOUT_VERSION 1

/* Limits: 1 <= N <= 2^30, 1 <= K <= W2A8_MAX_K, 1 <= M <= 2^20.  The K bound
 * keeps every int32 partial sum exact (|partial| <= 2048*K < 2^31). */
#define W2A8_MAX_K 1048448

/* Human-readable name of a status code (static string, never NULL). */
const char *w2a8_status_str(int status);

/* W2A8_LAYOUT_VERSION of the library (to check against the header). */
int w2a8_layout_version(void);

/* ------------------------------------------------------------------------
 * Packed weight layout "T32x128", version 1.
 *
 * [CPU] §2.1 maps -1 -> 00, 0 -> 01, 1 -> 10 (code = w + 1; 11 never
 * occurs) and [CPU] §2.2 stores 8 ternary weights in 2 bytes.  [TEST]
 * "编译 W2A8 CUDA 内核" describes the reference GPU kernel's block reorder
 * and 16-codes-per-32-bit-word interleave without giving the arrangement;
 * this arrangement is this library's own, chosen so that one wave64 reads
 * one 1 KiB tile with a single 16-byte load per lane:
 *
 *   Np = ceil(N/32)*32, Kp = ceil(K/128)*128, KT = Kp/128.
 *   Size: Np*Kp/4 bytes (exactly N*K/4 when N%32 == 0 and K%128 == 0).
 *   Tile (s, t) = rows 32s..32s+31, k 128t..128t+127, at byte (s*KT+t)*1024;
 *   the tiles of a 32-row strip are contiguous, strips follow each other.
 *   Inside a tile, lane slot l = 8*rg + kg (rg, kg in 0..7) is 16 bytes at
 *   offset 16*l: four little-endian 32-bit words q = 0..3, word q holding
 *   row 32s + 4rg + q at k = 128t + 16kg + i, i = 0..15.
 *   Inside a word, the code of i = 4j + b sits at bits 8b+2j .. 8b+2j+1, so
 *   (word >> 2j) & 0x03030303 holds the codes of k = 4j..4j+3 in bytes 0..3.
 *   Positions with row >= N or k >= K hold code 01 (weight 0).
 * ------------------------------------------------------------------------ */

/* Bytes of the packed matrix, or -1 if N or K is out of range. */
int64_t w2a8_packed_bytes(int64_t N, int64_t K);

/* Device workspace bytes that w2a8_gemv / w2a8_gemm need for (M, N, K),
 * or -1 if out of range.  For M = 1 it holds one 64-bit word per row, padded
 * to 32 rows (the tile count and partial sum of a row whose k-range is split
 * over several workgroups), and is 0 when no launch plan splits a k-range of
 * that K (with the default knobs: K <= 47*128 = 6016), whatever the device;
 * the M = 1 entry points then accept a NULL workspace.  For 2 <= M <= 32,
 * the larger of one such word per (row, padded output) and the split-K
 * space below; for M > 32, int32 partial sums and arrival counters of
 * split-K output blocks (0 bytes when M*N is too large for split-K, which is
 * then not used).  The caller allocates it,
 * zeroes it ONCE before its first use, and may then reuse it for any call
 * whose w2a8_workspace_bytes is no larger: each call leaves it zeroed
 * again. */
int64_t w2a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* ------------------------------------------------------------------------
 * Offline host steps
 * ------------------------------------------------------------------------ */

/* Absmean ternarization, host memory to host memory.
 * [WIN] §3.1 and [CPU] §6.3:  sw = mean(|W|);  wq = clamp(round(W/sw), -1, 1).
 * W: fp32 [N][K] row-major (host).  wq: int8 [N][K] (host).  sw: one float.
 * The mean is accumulated in fp64 in row-major order and rounded once to
 * fp32; W/sw is an fp32 division rounded half to even.  An all-zero W
 * gives sw = 0 and wq = 0.  Returns W2A8_ERR_NULL / W2A8_ERR_SHAPE. */
int w2a8_ternarize_absmean(const float *W, int64_t N, int64_t K, int8_t *wq,
                           float *sw);

/* Pack ternary weights into the T32x128 layout, host memory to host memory.
 * w: int8 [N][K] row-major with values in {-1, 0, 1}.  packed: at least
 * w2a8_packed_bytes(N, K) bytes (packed_bytes is its capacity).
 * Returns W2A8_ERR_VALUE if a weight is outside {-1, 0, 1} (packed is then
 * partly written and must not be used), W2A8_ERR_BUFSIZE if packed_bytes is
 * too small. */
int pack_ternary(const int8_t *w, int64_t N, int64_t K, void *packed,
                 int64_t packed_bytes);

/* Inverse of pack_ternary (host), for tests and inspection.  Returns
 * W2A8_ERR_VALUE if a code 11 is found at a position inside the matrix. */
int unpack_ternary(const void *packed, int64_t packed_bytes, int64_t N,
                   int64_t K, int8_t *w);

/* ------------------------------------------------------------------------
 * Device steps (enqueued on `stream`)
 * ------------------------------------------------------------------------ */

/* Per-token absmax quantization of bf16 activations to int8.
 * [TEST] (introduction): the kernels consume 8-bit activations; the pages
 * give no quantizer formula.  Per row m:
 *   a = max_k |x[m][k]|;  inv = min(127 / a, FLT_MAX)  (fp32 division; the cap
 *   only acts when a < 127 / FLT_MAX, where the quotient overflows);
 *   x_q[m][k] = clamp(round_half_even(x[m][k] * inv), -127, 127);
 *   s_a[m] = a / 127  (fp32 division).   A zero row gives 0 and s_a = 0.
 * x_bf16: device, [M][K] bf16 bit patterns (uint16), 16-byte aligned.
 * x_q: device, int8 [M][K], 16-byte aligned.  s_a: device, fp32 [M].
 * NaN and Inf inputs are outside the contract. */
int quant_act_int8(const uint16_t *x_bf16, int64_t M, int64_t K, int8_t *x_q,
                   float *s_a, void *stream);

/* W2A8 GEMV, M = 1 (decode).
 * [TEST] "运行 test.py 做 GEMV 基准测试" / "如何判断结果": y must equal the
 * integer product of the int8 activations and the weights exactly:
 *   y_i32[n] = sum_k w[n][k] * x[k]
 * [WIN] §3.1: the scale is multiplied back after the integer product:
 *   y_f32[n] = ((float)y_i32[n] * s_a[0]) * s_w
 * w_packed: device, T32x128 layout of W [N][K] (w2a8_packed_bytes(N, K)).
 * x: device, int8 [K].  y_i32: device, int32 [N], or NULL.  y_f32: device,
 * fp32 [N], or NULL; at least one of y_i32 / y_f32 must be given.  s_a:
 * device, one float (required when y_f32 is given; may be NULL otherwise).
 * s_w: the per-tensor weight scale, by value.  workspace: device, at least
 * w2a8_workspace_bytes(1, N, K) bytes, zeroed before first use (see above);
 * it may be NULL (and ws_bytes anything) when that size is 0.
 * Unlike the reference kernel, which computes only a fixed list of shapes
 * ([TEST] "限制与注意事项"), every N, K within the limits is computed. */
int w2a8_gemv(const void *w_packed, const int8_t *x, int64_t N, int64_t K,
              int32_t *y_i32, const float *s_a, float s_w, float *y_f32,
              void *workspace, int64_t ws_bytes, void *stream);

/* Static scratch of w2a8_gemv_noalloc, in bytes (per device). */
#define W2A8_NOALLOC_SCRATCH_BYTES (1 << 20)

/* w2a8_gemv without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments (minus workspace and ws_bytes), the
 * same plans and kernels, bit-identical results.  Where w2a8_gemv would use
 * its workspace (w2a8_workspace_bytes(1, N, K) > 0), this call uses a
 * static device array of the library of W2A8_NOALLOC_SCRATCH_BYTES bytes per
 * device (one 64-bit word per padded output row: N up to 131072 rows then),
 * held until the process ends; larger N is rejected with W2A8_ERR_SCRATCH
 * before any device work.  The call allocates nothing.  The array is zero
 * when the library loads and every complete call leaves it zero; the first
 * call on a device also clears it with a small kernel on `stream` when the
 * stream is not capturing.  Every call on one device shares the one array:
 * calls that may overlap on a device (other streams, other host threads)
 * race and must not be issued. */
int w2a8_gemv_noalloc(const void *w_packed, const int8_t *x, int64_t N, int64_t K,
                      int32_t *y_i32, const float *s_a, float s_w, float *y_f32,
                      void *stream);

/* Whole linear layer for one token, in one launch: the result of
 * quant_act_int8 (M = 1) followed by w2a8_gemv with its fp32 epilogue,
 * bit-identical to that pair.
 * [WIN] §3.1: integer product of the quantized activations and the ternary
 * weights, the scales multiplied back afterwards; [TEST] (introduction):
 * 8-bit activations.  Every workgroup takes the row maximum itself, so the
 * quantized row never goes through memory (it reads the bf16 row once per
 * workgroup from the L2).
 * x_bf16: device, bf16 [K] bit patterns, 16-byte aligned.  y_f32: device,
 * fp32 [N] (required).  y_i32: device, int32 [N] of the integer product, or
 * NULL.  s_w, workspace, ws_bytes, stream: as w2a8_gemv. */
int w2a8_linear_gemv(const void *w_packed, const uint16_t *x_bf16, int64_t N, int64_t K,
                     float s_w, float *y_f32, int32_t *y_i32, void *workspace,
                     int64_t ws_bytes, void *stream);

/* Most projections in one grouped call. */
#define W2A8_MAX_GROUPS 8

/* Several decode GEMVs that share the activation row and K, in one launch
 * (for example a layer's query, key and value projections, or its gate and
 * up projections).  For each projection g the result is exactly that of
 *   w2a8_gemv(w_packed[g], x, N[g], K, y_i32[g], s_a, s_w[g], y_f32[g], ...):
 *   y_i32[g][n] = sum_k w_g[n][k] * x[k]
 *   y_f32[g][n] = ((float)y_i32[g][n] * s_a[0]) * s_w[g]
 * ([TEST] "运行 test.py 做 GEMV 基准测试" / "如何判断结果" for the exact
 * integer product, [WIN] §3.1 for the scales).  One launch instead of G
 * saves the launch gaps and fills the device with the projections' strips
 * together.
 * G: 1 <= G <= W2A8_MAX_GROUPS.  w_packed, N, s_w: HOST arrays of G entries,
 * read during the call only; w_packed[g] is a device T32x128 buffer of
 * W_g [N[g]][K] (16-byte aligned).  y_i32, y_f32: HOST arrays of G device
 * pointers, or NULL for no outputs of that kind; single entries may be NULL,
 * but every projection needs at least one output.  x, s_a: as w2a8_gemv
 * (s_a required when any y_f32 entry is given).  The padded rows
 * (sum_g N[g] rounded up to 32 each) must not exceed 2^30.  workspace:
 * device, at least sum_g w2a8_workspace_bytes(1, N[g], K) bytes, zeroed
 * before first use (NULL when that sum is 0).  Errors: W2A8_ERR_SHAPE for G or an N[g] out of range,
 * otherwise as w2a8_gemv. */
int w2a8_gemv_grouped(int G, const void *const *w_packed, const int64_t *N, int64_t K,
                      const int8_t *x, const float *s_a, const float *s_w,
                      int32_t *const *y_i32, float *const *y_f32, void *workspace,
                      int64_t ws_bytes, void *stream);

/* Grouped form of w2a8_linear_gemv: quantize the bf16 row (as
 * quant_act_int8, M = 1) and apply G projections sharing it, in one launch;
 * bit-identical to quant_act_int8 followed by w2a8_gemv_grouped.
 * y_f32: HOST array of G device pointers, all required.  y_i32: HOST array
 * of G device pointers (entries may be NULL), or NULL.  Other arguments as
 * w2a8_gemv_grouped and w2a8_linear_gemv. */
int w2a8_linear_gemv_grouped(int G, const void *const *w_packed, const int64_t *N, int64_t K,
                             const uint16_t *x_bf16, const float *s_w, float *const *y_f32,
                             int32_t *const *y_i32, void *workspace, int64_t ws_bytes,
                             void *stream);

/* ------------------------------------------------------------------------
 * W2A4 variant: int4 activations.
 * "使用 BitNet 框架部署 1-bit LLM：三元权重量化、LUT 矩阵乘加速与 GPU 运行时优化",
 * section "GPU 运行时优化与低延迟推理管道", names an "a4.8" extension with
 * lower-precision activations, without a formula.
 * Reading: the per-token absmax quantizer above with 7 levels per side, and
 * the same exact integer product and fp32 epilogue.
 *
 * Activation layout "A4I": a row of K values padded with zeros to
 * Kq = ceil(K/32)*32 values, two's complement nibbles, Kq/2 bytes per row,
 * rows back to back.  Value k: chunk c = k/16, i = k%16, h = i/4, j = i%4;
 * byte c*8 + 4*(h%2) + j, low nibble for h < 2, high nibble otherwise.  (Byte
 * j of a chunk's first word holds values j and 8+j, of its second word
 * values 4+j and 12+j: the positions of their weight codes in a T32x128 word
 * under the masks 0x33333333 and (w >> 2) & 0x33333333.)
 * ------------------------------------------------------------------------ */

/* Bytes of M rows of K int4 activations in the A4I layout, or -1 for M or K
 * out of range. */
int64_t w2a4_act_bytes(int64_t M, int64_t K);

/* Host: pack int4 values q (int8 [M][K], each in -8..7) into the A4I layout
 * (out: host, out_bytes >= w2a4_act_bytes(M, K)).  W2A8_ERR_VALUE for a value
 * outside -8..7 (out then partly written). */
int pack_act_int4(const int8_t *q, int64_t M, int64_t K, uint8_t *out, int64_t out_bytes);

/* Per-token absmax int4 quantization of bf16 activations (device).  Per row m:
 *   a = max_k |x[m][k]|;  inv = min(7 / a, FLT_MAX)  (fp32 division; the cap
 *   only acts when a < 7 / FLT_MAX);
 *   q[m][k] = clamp(round_half_even(x[m][k] * inv), -7, 7);
 *   s_a[m] = a / 7  (fp32 division).   A zero row gives 0 and s_a = 0.
 * x_bf16: device, [M][K] bf16 bit patterns, 16-byte aligned.  x_q4: device,
 * w2a4_act_bytes(M, K) bytes, 16-byte aligned, written in the A4I layout
 * (padding nibbles zero).  s_a: device, fp32 [M]. */
int quant_act_int4(const uint16_t *x_bf16, int64_t M, int64_t K, uint8_t *x_q4,
                   float *s_a, void *stream);

/* W2A4 GEMV, M = 1: w2a8_gemv with int4 activations.
 *   y_i32[n] = sum_k w[n][k] * q[k]
 *   y_f32[n] = ((float)y_i32[n] * s_a[0]) * s_w
 * x_q4: device, one A4I row (w2a4_act_bytes(1, K) bytes), 16-byte aligned.
 * Every other argument as w2a8_gemv (same packed weights, same workspace
 * size w2a8_workspace_bytes(1, N, K)). */
int w2a4_gemv(const void *w_packed, const uint8_t *x_q4, int64_t N, int64_t K,
              int32_t *y_i32, const float *s_a, float s_w, float *y_f32,
              void *workspace, int64_t ws_bytes, void *stream);

/* W2A4 linear layer for one token, in one launch: the result of
 * quant_act_int4 (M = 1) followed by w2a4_gemv with its fp32 epilogue,
 * bit-identical to that pair.  Every workgroup takes the row maximum and
 * quantizes the part of the row its waves consume into LDS, so the int4 row
 * never goes through memory.
 * x_bf16: device, bf16 [K] bit patterns, 16-byte aligned.  y_f32: device,
 * fp32 [N] (required).  y_i32: device, int32 [N] of the integer product, or
 * NULL.  w_packed, N, K, s_w, workspace, ws_bytes, stream: as w2a4_gemv
 * (same workspace size). */
int w2a4_linear_gemv(const void *w_packed, const uint16_t *x_bf16, int64_t N, int64_t K,
                     float s_w, float *y_f32, int32_t *y_i32, void *workspace,
                     int64_t ws_bytes, void *stream);

/* W2A8 batched product, M >= 1 (prefill).
 * [TEST] "限制与注意事项": the reference handles only M == 1; this entry
 * computes the same product for M token rows:
 *   y_i32[m][n] = sum_k w[n][k] * x[m][k]
 *   y_f32[m][n] = ((float)y_i32[m][n] * s_a[m]) * s_w
 * x: device, int8 [M][K].  y_i32 / y_f32: device, [M][N] (at least one).
 * s_a: device, fp32 [M] (required with y_f32).  workspace: at least
 * w2a8_workspace_bytes(M, N, K) bytes, zeroed before first use. */
int w2a8_gemm(const void *w_packed, const int8_t *x, int64_t M, int64_t N,
              int64_t K, int32_t *y_i32, const float *s_a, float s_w,
              float *y_f32, void *workspace, int64_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W2A8_H */
