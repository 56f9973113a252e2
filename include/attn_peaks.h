/*
 * attn_peaks.h -- measured ceilings of the GPU for the benchmark's roofline
 * fractions (libattn_peaks.so; not part of the attention library).
 *
 * attn_peak_mfma_bf16        enqueue `workgroups` workgroups of 4 waves, each
 *                            wave issuing `iters` rounds of 4 independent
 *                            32x32x16 bf16 matrix-core products (fp32
 *                            accumulate).  `out`: device float array of
 *                            workgroups*256 entries (written).  Returns 0,
 *                            -1 for a bad argument, -4 for a failed launch.
 * attn_peak_mfma_bf16_flops  the flops one such launch performs.
 * attn_peak_stream_read      enqueue a non-temporal streaming read of the
 *                            first `bytes` (rounded down to 16) of the device
 *                            buffer `src` (16-byte aligned) by `workgroups`
 *                            workgroups; `out` is a device uint32 that is
 *                            written only in a case that never happens in
 *                            practice (keeps the loads live).  Same returns.
 * Both take a hipStream_t (NULL: default stream) and return once enqueued;
 * the caller times them with events on that stream.
 */
#ifndef ATTN_PEAKS_H
#define ATTN_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int attn_peak_mfma_bf16(int iters, int workgroups, float *out, void *hip_stream);
double attn_peak_mfma_bf16_flops(int iters, int workgroups);
int attn_peak_stream_read(const void *src, size_t bytes, uint32_t *out, int workgroups,
                          void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PEAKS_H */
