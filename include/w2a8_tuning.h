/*
 * w2a8_tuning.h — launch-shape knobs of libw2a8.so, for measurement sweeps.
 *
 * Not needed for normal use: the defaults are the measured best on MI355X.
 * The knobs are process-wide (not per device) and are read when a call is
 * made; change them only while no other host thread is calling the library.
 */
#ifndef W2A8_TUNING_H
#define W2A8_TUNING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GEMV launch plan (w2a8_gemv).  A 32-row strip with at least
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

/* Streaming GEMV for large matrices: used when the matrix has at least
 * `min_tiles` 1 KiB tiles (0: never, the default) and 16 <= K <= 32768 (all
 * activations fit in LDS).  The grid is CUs * `waves_per_cu` (1..64) long-lived waves, each
 * streaming an equal contiguous share of the tiles with two load batches of
 * `unroll` (2, 4 or 8) tiles in flight.  Returns W2A8_OK or W2A8_ERR_VALUE. */
int w2a8_tune_gemv_stream(int min_tiles, int waves_per_cu, int unroll);

/* Batched product kernel (w2a8_gemm): 0 = automatic (default), 1 = the
 * pipelined MFMA kernel whenever K is a multiple of 16 (its configuration
 * still chosen by shape, including the wave-group k-split for small output
 * grids; it never splits K across workgroups), 2 = the general kernel
 * (split-K across workgroups for small outputs) always, 3 = the few-row
 * kernel (GEMV-style, dot4 on decoded weights) whenever M <= 8, the
 * automatic choice above that.  The automatic
 * rule, from measurements on MI355X: the few-row kernel for
 * M <= 2 up to 49152 weight tiles and for K not a multiple of 16 (M <= 8);
 * the general kernel for K not a multiple of 16 above that; otherwise the
 * pipelined kernel.  Returns W2A8_OK or W2A8_ERR_VALUE. */
int w2a8_tune_gemm(int kernel);

/* The plan w2a8_gemv would use for (N, K) on a device with `cus` compute
 * units under the current knobs.  Streaming kernel: *stream_waves = grid
 * waves, *unroll = its batch, the other outputs 0.  Otherwise *stream_waves
 * = 0 and waves per workgroup, workgroups per strip and load batch of the
 * workgroup-split kernel.  Returns W2A8_OK, W2A8_ERR_NULL or
 * W2A8_ERR_SHAPE. */
int w2a8_gemv_plan(int64_t N, int64_t K, int cus, int *waves_per_wg, int *wgs_per_strip,
                   int *unroll, int *stream_waves);

#ifdef __cplusplus
}
#endif

#endif /* W2A8_TUNING_H */
