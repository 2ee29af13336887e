/*
 * ssm_decode.h -- C ABI of the fused decode step of a Mamba block: the depthwise causal
 * conv1d step followed by the selective-scan step, for one token, in one launch.
 *
 * Source: the decode path of the Mamba block in mamba-rs kernels.rs (MambaKernels
 * fields conv1d_step and ssm_step_fwd, run one after the other for each generated
 * token); the conv1d step is the depthwise causal convolution of the block's x branch
 * (width K window of the previous K - 1 inputs and the new one, bias, SiLU), the scan
 * step the selective-scan recurrence at L = 1.
 *
 * ssm_decode_step computes, for each (b, d):
 *   u[b,d]      = act(bias[d] + sum_{k<K} weight[d,k] * window[k]),
 *                 window = (conv_state[b,d,0..K-2], x[b,d]); act = SiLU or identity
 *   conv_state  <- (window[1..K-1])                    (shifted in place)
 *   then exactly ssm_scan_step_ex on x := u (u rounded to io_dtype first, as a separate
 *   ssm_conv1d_step would store it): state updated in place, y written.
 * The results are bit-identical to ssm_conv1d_step followed by ssm_scan_step_ex with the
 * same arguments (u as the scan's x).
 *
 * Arguments:
 *   conv_state  : [batch, d_inner, width-1] io_dtype, read and written (NULL iff width == 1)
 *   x           : [batch, d_inner] io_dtype, the token before the convolution
 *   conv_weight : [d_inner, width] fp32; conv_bias: [d_inner] fp32, nullable (zero)
 *   width       : 1..8; activation: SSM_ACT_NONE or SSM_ACT_SILU (ssm_conv1d.h)
 *   state, delta_raw, z, B, C, A_log, D_skip, dt_bias, y, d_state, options: as for
 *               ssm_scan_step_ex (ssm_scan.h)
 *   u           : [batch, d_inner] io_dtype, the convolution's output, nullable (not written)
 * Layout: row-major, last index fastest.  Ownership: the caller allocates every buffer;
 * nothing is allocated.  Work is enqueued on `stream`; the call does not wait.
 * Errors (nothing is launched): SSM_ERR_NULL (a required pointer is NULL), SSM_ERR_DIM,
 * SSM_ERR_UNSUPPORTED (io_dtype, activation), SSM_ERR_ARG (options), SSM_ERR_ALIGN
 * (pointers not aligned to their element size), SSM_ERR_ALIAS (an output overlaps an
 * input or another output); a launch failure is SSM_ERR_HIP.
 */
#ifndef SSM_DECODE_H
#define SSM_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "ssm_conv1d.h"
#include "ssm_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

int ssm_decode_step(void* conv_state, const void* x, const float* conv_weight, const float* conv_bias,
                    int64_t width, int activation, float* state, const void* delta_raw, const void* z,
                    const void* B, const void* C, const float* A_log, const float* D_skip,
                    const float* dt_bias, void* u, void* y, int64_t batch, int64_t d_inner, int64_t d_state,
                    int io_dtype, const ssm_scan_options* options, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_DECODE_H */
