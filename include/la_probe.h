/*
 * la_probe.h -- peak probes of libla_probe.so (not part of the operator's ABI).
 *
 * Measurement tools for the roofline denominators: what one GPU sustains
 * for a streaming copy and for bf16 matrix-core work.  Every pointer is a
 * device pointer owned by the caller; calls are asynchronous on `stream`
 * (a hipStream_t, NULL = null stream) and return 0 on success, 1 on a bad
 * argument (nothing launched), 3 when the launch failed.
 */
#ifndef LA_PROBE_H
#define LA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` (a multiple of 16; both pointers 16-byte aligned, not
 * overlapping) from src to dst: every byte is read once and written once. */
int la_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

/* `blocks` workgroups of four waves, each wave issuing `iters` steps of four
 * independent v_mfma_f32_32x32x16_bf16 products on register operands; writes
 * blocks * 256 floats to `out` (float32, keeps the results live). */
int la_probe_mfma(float *out, int blocks, int iters, void *stream);

/* Matrix flops one la_probe_mfma(blocks, iters) launch performs. */
double la_probe_mfma_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* LA_PROBE_H */
