/*
 * ust_calib.h - measurement aids exported by the same library as ust.h.
 *
 * Not steps of the attention path: a kernel that only issues bf16 MFMAs, so
 * that a benchmark can report the matrix rate the part sustains under load
 * beside the published peak, and compare each kernel with both.  The shader
 * clock under a matrix load is power-limited and the power depends on the
 * operands' bits, so the kernel feeds pseudo-random operands (random signs
 * and mantissas, magnitude 0.5 .. 2), as a kernel on real data would see.  Same conventions as ust.h:
 * caller-owned device memory, asynchronous on `stream`, validation before
 * launch, status codes and ust_last_error().
 */
#ifndef UST_CALIB_H
#define UST_CALIB_H

#include "ust.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launch n_workgroups workgroups of 8 waves; every wave issues
 * iters x 4 independent v_mfma_f32_32x32x16_bf16 back to back, on four
 * pseudo-random operand pairs in turn, and writes one fp32 sum to
 * out[workgroup * 8 + wave].
 *   out: fp32 [n_workgroups * 8], written (the values carry no meaning).
 *   flops_out: host pointer or NULL; receives the launch's flop count,
 *              n_workgroups * 8 * iters * 4 * 32768.
 * Errors: out NULL (UST_E_NULL); n_workgroups or iters not positive, or
 * n_workgroups above 65536 (UST_E_SHAPE); out misaligned (UST_E_ALIGN). */
ust_status ust_calib_mfma_bf16(int32_t n_workgroups, int32_t iters, float* out,
                               double* flops_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* UST_CALIB_H */
