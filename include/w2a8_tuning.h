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

/* GEMV work split (w2a8_gemv).  Each 32-row strip of the packed matrix is
 * cut into S contiguous k-parts, one wave each, with S the smallest count
 * that gives about `waves_per_cu` waves per compute unit but no part
 * shorter than `min_tiles` 1 KiB tiles.  `unroll` (2, 4 or 8) is the number
 * of 16-byte loads each lane keeps in flight.  Returns W2A8_OK or
 * W2A8_ERR_VALUE for out-of-range knobs (1..64, >= 1, {2,4,8}). */
int w2a8_tune_gemv(int waves_per_cu, int min_tiles, int unroll);

/* The k-parts per strip S that w2a8_gemv would use for (N, K) on a device
 * with `cus` compute units under the current knobs (-1 if out of range). */
int w2a8_gemv_split(int64_t N, int64_t K, int cus);

#ifdef __cplusplus
}
#endif

#endif /* W2A8_TUNING_H */
