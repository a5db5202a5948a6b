/*
 * orbitquant_diag.h -- diagnostic entry points of liborbitquant.so, used to
 * measure the ceilings the path's kernels are compared with.  Not part of
 * the quantized-linear path; same conventions as orbitquant.h (status
 * codes, validation before any HIP call, asynchronous on `stream`).
 */
#ifndef ORBITQUANT_DIAG_H
#define ORBITQUANT_DIAG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core throughput probe: `blocks` workgroups of 512 threads; every
 * wave issues `iters` rounds of 32 independent v_mfma_f32_16x16x32_f16
 * (fp16 operands, fp32 accumulation), nothing else in the loop.  Work:
 * blocks * 8 * iters * 32 * 16384 flop.  The caller times the launch.
 *   sink: device fp32 [blocks * 512], receives one sum per thread so the
 *         work cannot be optimised away (values are meaningless)
 * blocks >= 1, iters >= 1.  Errors: OQ_EINVAL (null sink, bad counts),
 * OQ_EDEVICE. */
int oq_diag_mfma_f16(int blocks, int iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* ORBITQUANT_DIAG_H */
