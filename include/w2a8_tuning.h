/*
 * w2a8_tuning.h — launch-shape knobs of libw2a8.so, for measurement sweeps.
 *
 * Not needed for normal use: the defaults are the measured best on MI355X.
 * The knobs are process-wide (not per device).  Setting them is thread-safe:
 * each device call takes one consistent copy of the knobs when it starts, so
 * a call running concurrently with a change uses either all old or all new
 * values (and every plan computes the same result).
 */
#ifndef W2A8_TUNING_H
#define W2A8_TUNING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GEMV launch plan of the batch kernel (w2a8_gemv for K not a multiple of
 * 16; the fused, grouped and W2A4 GEMVs).  The ring kernel's plan uses only
 * `split_min_tiles` (the shortest strip it splits over workgroups).  A
 * 32-row strip with at least
 * `split_min_tiles` k-tiles (1 KiB each) is split over workgroups: about one
 * per `tiles_per_wave` tiles, at most 12, and more when there are too few
 * strips to give `wg_per_cu` (1..64) workgroups per compute unit; never more
 * than `krange_tiles` (1..256) tiles per workgroup.  Split strips combine
 * their partial sums through the workspace.  A workgroup splits its k-range
 * over up to 16 waves with runs of about `tiles_per_wave` tiles (1..32).
 * Each wave keeps two load batches in flight; a batch is the smallest of 2,
 * 4, 8 tiles whose two batches cover the run, but at most `unroll` (2, 4 or
 * 8).  Defaults: (4, 6, 8, 256, 48).  Returns W2A8_OK or W2A8_ERR_VALUE for
 * out-of-range knobs. */
int w2a8_tune_gemv(int wg_per_cu, int tiles_per_wave, int unroll, int krange_tiles,
                   int split_min_tiles);

/* Forced GEMV plan for measurement sweeps (w2a8_gemv only; the fused,
 * grouped and W2A4 GEMVs keep their automatic plans).  kernel 0 restores the
 * automatic plan (other arguments ignored).  kernel 1: the batch kernel with
 * `waves_per_wg` (1..16) waves per workgroup, `wgs_per_strip` (1..4096)
 * workgroups per 32-row strip (at most one per k-tile), two load batches of
 * `depth` (2, 4 or 8) tiles, and each tile's activations loaded next to its
 * weights when `direct_x` is 1 (K a multiple of 16; not with batch 8) instead
 * of staging the wave's run in LDS.  kernel 2: the ring kernel (K a multiple
 * of 16) with `depth` (2, 4, 6, 8 or 12) tiles in flight per wave; it always
 * loads activations next to the weights, so `direct_x` must be 1.  kernel 3:
 * the row-slice kernel (K a multiple of 16): 8 single-wave workgroups per
 * strip, each owning 4 of the 32 rows of every tile, with `depth` (2, 4, 6
 * or 8) steps of 8 tiles in flight; it never splits the k-range, so
 * `waves_per_wg` must be 1, `wgs_per_strip` 8 and `direct_x` 1.
 * w2a8_gemv returns W2A8_ERR_VALUE for a forced batch plan whose runs exceed
 * 32 tiles per wave, or a forced ring or row-slice plan on K not a multiple
 * of 16.  w2a8_workspace_bytes(1, N, K) counts a forced split.  Returns W2A8_OK or
 * W2A8_ERR_VALUE. */
int w2a8_tune_gemv_force(int kernel, int waves_per_wg, int wgs_per_strip, int depth,
                         int direct_x);

/* Batched product kernel (w2a8_gemm): 0 = automatic (default), 1 = the
 * pipelined MFMA kernel whenever K is a multiple of 16 (its configuration
 * still chosen by shape, including the wave-group k-split for small output
 * grids; it never splits K across workgroups), 2 = the general kernel
 * (split-K across workgroups for small outputs) always, 3 = the few-row
 * kernel (GEMV-style, dot4 on decoded weights) whenever M <= 8, 4 = the
 * short-batch MFMA ring kernel (the GEMV's weight stream feeding int8 MFMA)
 * whenever M <= 32 and K is a multiple of 16; other shapes take the
 * automatic choice.  The automatic rule, from measurements on MI355X: the
 * few-row kernel for M <= 2 up to 49152 weight tiles and for K not a multiple
 * of 16 (M <= 8); the ring kernel for the other M <= 8, for 9 <= M <= 16
 * with fewer than 3 weight strips (of 32 rows) per compute unit, and for
 * 17 <= M <= 32 with K of at least 192 tiles of 128 over fewer strips than
 * compute units; the general kernel for K not a multiple of 16 above that;
 * otherwise the pipelined kernel.
 * Returns W2A8_OK or W2A8_ERR_VALUE. */
int w2a8_tune_gemm(int kernel);

/* Measurement knob: force configuration `config` (0..9) of the pipelined
 * MFMA GEMM's table (workgroup rows, waves, strips per wave, ring stages and
 * wave groups over K) wherever w2a8_gemm takes the pipelined kernel; -1
 * restores the automatic choice.  Every configuration computes every shape
 * exactly; only speed differs.  Returns W2A8_OK or W2A8_ERR_VALUE. */
int w2a8_tune_gemm_pipe(int config);

/* Forced plan of the short-batch MFMA ring kernel, wherever w2a8_gemm takes
 * it: `waves_per_wg` (1..16) waves per workgroup splitting a 32-row strip's
 * k-range, `wgs_per_strip` (1..4096; at most the strip's k-tiles are used)
 * workgroups per strip, `depth` (2, 4, 6 or 8) tiles in flight per wave.
 * All three 0 restore the automatic plan.  w2a8_gemm returns W2A8_ERR_VALUE
 * for a forced plan whose rings need more LDS than a workgroup may allocate
 * on the device.  Returns W2A8_OK or W2A8_ERR_VALUE. */
int w2a8_tune_gemm_ring(int waves_per_wg, int wgs_per_strip, int depth);

/* The automatic plan w2a8_gemv would use for (N, K) on a device with `cus`
 * compute units under the current knobs: the kernel (3: the row-slice kernel,
 * for K a multiple of 16 on matrices of small packed size: at most cus/2
 * strips of at most 64 k-tiles, or 96 from cus/4 strips, or at most cus
 * strips of 48 to 64 k-tiles;
 * 2: the ring kernel, for the other K multiples of 16; 1: the batch kernel,
 * for other K), waves per workgroup, workgroups per 32-row strip (kernel 3:
 * always 8 row slices, no split; kernels 1 and 2: k-ranges, more than 1 only
 * when w2a8_workspace_bytes(1, N, K) > 0) and depth (ring: tiles in flight
 * per wave; row-slice: steps of 8 tiles in flight; batch: load batch).
 * Returns W2A8_OK, W2A8_ERR_NULL or W2A8_ERR_SHAPE. */
int w2a8_gemv_plan(int64_t N, int64_t K, int cus, int *kernel, int *waves_per_wg,
                   int *wgs_per_strip, int *depth);

/* The automatic plan of the fused linear layer for one token
 * (w2a8_linear_gemv with int4 = 0, w2a4_linear_gemv with int4 = 1) for
 * (N, K) on a device with `cus` compute units under the current knobs.
 * kernel: 1 the workgroup kernel's fused variant (int8 only), 3 the ring
 * kernel over shared k-ranges (*waves_per_wg strips per workgroup, one wave
 * each, quantizing one k-range of at most *run tiles into LDS), 4 the ring
 * kernel with per-wave runs (int4 only: *waves_per_wg waves per strip, runs
 * of at most *run tiles, each quantized into its own LDS region).
 * *wgs_per_strip: k-ranges per strip (more than 1 only when
 * w2a8_workspace_bytes(1, N, K) > 0).  *depth: ring depth, or the load batch
 * of kernel 1.  Returns W2A8_OK, W2A8_ERR_NULL or W2A8_ERR_SHAPE. */
int w2a8_linear_plan(int64_t N, int64_t K, int cus, int int4, int *kernel, int *waves_per_wg,
                     int *wgs_per_strip, int *run, int *depth);

#ifdef __cplusplus
}
#endif

#endif /* W2A8_TUNING_H */
