/*
 * serq_peaks.h -- sustained-rate probes of MI355X (gfx950) that the SERQ
 * layer's roofline fractions are read against (libserq_peaks.so).  Published
 * peaks assume one MFMA per pipeline slot on every SIMD at the nominal clock;
 * these measure what the chip sustains under the same instructions.
 *
 * Every call enqueues one kernel on `stream` (a hipStream_t, NULL = default)
 * and returns 0, or -1 for an invalid argument (nothing launched), or -5 for
 * a HIP launch error.  Buffers are device memory owned by the caller; the
 * caller times the launches (e.g. HIP events on the same stream).
 */
#ifndef SERQ_PEAKS_H
#define SERQ_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Floats the MFMA probe's sink needs for waves_per_simd (1 or 2) on the
 * current device: one per thread of one workgroup per compute unit. */
int serq_peak_sink_floats(int waves_per_simd);

/* Rate of the constant wall clock the MFMA probe records, in kHz (0 if the
 * device does not report it). */
int serq_peak_wall_khz(void);

/* One workgroup per compute unit of 256 (waves_per_simd = 1) or 512 (= 2)
 * threads; every wave runs iters x 8 MFMAs on 8 independent accumulators
 * with register operands.  kind: 0 = v_mfma_i32_16x16x64_i8 (32768 ops
 * each), 1 = scaled 16x16x128 FP4 x FP4, 2 = FP8 x FP8, 3 = FP4 x FP8 (65536
 * flops each).  sink: device float[serq_peak_sink_floats(waves_per_simd)]
 * (the accumulators' sums, so no MFMA is dead); clocks: device int64[2],
 * written by the first wave: shader-clock cycles and wall-clock ticks (rate:
 * hipDeviceAttributeWallClockRate) of its loop. */
int serq_peak_mfma(int kind, int waves_per_simd, int iters, float *sink, long long *clocks, void *stream);

/* Reads `bytes` (a multiple of 16, 16-byte aligned) of src in 16-byte pieces
 * at a grid stride; sink: device uint32[8 * 256 * compute units]. */
int serq_peak_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Copies `bytes` (a multiple of 16, both 16-byte aligned) from src to dst. */
int serq_peak_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SERQ_PEAKS_H */
