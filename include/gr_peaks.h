/*
 * gr_peaks.h -- C ABI of the measurement probes (libgr_peaks.so): the
 * sustained rates of one gfx950 that the benchmark reports beside the
 * vendor peaks (the roofline fractions use the vendor peaks).  These calls
 * are not part of the decode path.
 *
 * Every entry point enqueues one kernel launch on `stream` (a hipStream_t;
 * NULL = the null stream) and returns its HIP status (0 = success).  A
 * non-positive size, grid or iteration count, or a NULL pointer, returns
 * hipErrorInvalidValue (1) and enqueues nothing.  All buffers are
 * caller-owned device memory; `grid` is the number of 256-thread
 * workgroups.
 */
#ifndef GR_PEAKS_H
#define GR_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Four independent chains of `iters` v_mfma_f32_32x32x16_bf16 per wave
 * (32768 flops each): grid*4*iters*4*32768 flops.  out: fp32 [grid*256]. */
int gr_peak_mfma(float *out, int grid, int iters, void *stream);

/* Eight independent chains of `iters` fp32 exp2 per thread:
 * grid*256*iters*8 results.  out: fp32 [grid*256]. */
int gr_peak_exp2(float *out, int grid, int iters, void *stream);

/* Streaming copy of n16 16-byte words from src to dst (no overlap). */
int gr_peak_copy(const void *src, void *dst, int64_t n16, int grid, void *stream);

/* Streaming read of n16 16-byte words of src; out: uint32 [grid*256]. */
int gr_peak_read(const void *src, int64_t n16, uint32_t *out, int grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GR_PEAKS_H */
