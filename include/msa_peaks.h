/*
 * msa_peaks.h -- measurement kernels in libmsa.so, not part of the method.
 *
 * The benchmark reports each kernel's achieved rate against MI355X's published
 * peaks (HBM3E 8 TB/s, bf16 dense MFMA 2.5 PFLOP/s).  These two kernels measure
 * what the device under test actually sustains, so the reports can show both
 * fractions: a streaming read of a large buffer (bytes per second from HBM)
 * and a loop of independent v_mfma_f32_16x16x32_bf16 chains (dense bf16
 * FLOP/s at the clock the chip holds under MFMA load).
 *
 * Both enqueue one kernel on `stream` (a hipStream_t; NULL = default stream),
 * allocate nothing and never synchronise; the caller times them (for example
 * with HIP events) and owns every buffer.  Errors are returned as the negative
 * msa_status codes of msa.h, with the message in msa_last_error().
 */
#ifndef MSA_PEAKS_H
#define MSA_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read every byte of buf (device memory, `bytes` > 0, a multiple of 16,
 * 16-byte aligned) once.  sink: device uint32 the kernel may write one value
 * to (so the reads cannot be elided); its contents are unspecified.
 * MSA_ERR_INVALID on a NULL, misaligned or badly sized buffer. */
int msa_peaks_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* The same read with its knobs exposed, for a sweep of the read rate:
 * `unroll` loads in flight per thread per iteration (1, 2, 4, 8 or 16), loads
 * of `width` bytes (4, 8 or 16), plain (nontemporal == 0) or nontemporal
 * loads, and at most wg_per_cu (1..64) workgroups of 256 threads per CU
 * (256 CUs), grid-striding over the buffer.  Arguments otherwise as
 * msa_peaks_stream_read; MSA_ERR_INVALID for a knob outside its set. */
int msa_peaks_stream_read_variant(const void *buf, int64_t bytes, uint32_t *sink, int32_t unroll, int32_t width,
                                  int32_t nontemporal, int32_t wg_per_cu, void *stream);

/* workgroups x 4 waves each run `iters` rounds of 4 independent 16x16x32 bf16
 * MFMAs: workgroups * 4 * iters * 4 * 16384 FLOP in total.  sink: device
 * float[256] the kernel may write to; contents unspecified.  workgroups in
 * [1, 2^20], iters in [1, 2^20]; MSA_ERR_INVALID otherwise. */
int msa_peaks_mfma(float *sink, int32_t workgroups, int32_t iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PEAKS_H */
