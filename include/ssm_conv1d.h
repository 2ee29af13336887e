/*
 * ssm_conv1d.h -- C ABI of the depthwise causal conv1d (+ optional SiLU) in
 * libssmscan.so: the step before the selective scan in a Mamba block.
 *
 * The operation, one filter of K taps per channel, no history before t = 0:
 *   p[b,t,d]   = sum_{k<K} weight[d,k] * x[b, t-(K-1)+k, d] + bias[d]
 *   out[b,t,d] = silu(p) when activation = SSM_ACT_SILU, p when SSM_ACT_NONE
 * Passages that define it: mamba-rs kernels.rs, MambaKernels conv1d fields
 * (conv1d_step_fwd, the one-step depthwise conv with SiLU used in decoding;
 * conv1d_burnin_fwd and _nosave, the multi-step forward; conv1d_step_bwd and
 * conv1d_burnin_bwd, their backward); deterministic_backward.py, ordered_conv
 * (training runs from reset sequences, without initial states; the weight and bias
 * gradients are fp32 sums of per-batch partials added in batch order).
 *
 * Conventions (as in ssm_scan.h: statuses, ownership, asynchrony, validation
 * before launch, determinism):
 *   Layouts, row-major, last index fastest:
 *     x, out, dout, dx : [batch, seqlen, dim] (a step: [batch, dim])
 *     weight, dweight  : [dim, width] fp32        bias, dbias : [dim] fp32
 *     conv_state       : [batch, dim, width-1] io_dtype, the width-1 most recent
 *                        inputs of each channel, oldest first
 *   io_dtype is the element type of x, out and conv_state (SSM_F32 or SSM_BF16;
 *   the backward is SSM_F32 only).  Arithmetic is fp32.
 *   Supported: 1 <= width <= 8; batch, seqlen, dim >= 1.
 */
#ifndef SSM_CONV1D_H
#define SSM_CONV1D_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "ssm_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSM_ACT_NONE = 0, SSM_ACT_SILU = 1 } ssm_activation;

/* Causal conv over whole sequences.  x, weight, out required; bias optional (NULL
 * means zero).  out must not overlap the inputs. */
int ssm_conv1d_fwd(const void* x, const float* weight, const float* bias, void* out, int64_t batch,
                   int64_t seqlen, int64_t dim, int64_t width, int activation, int io_dtype,
                   hipStream_t stream);

/* One decode step: window = (conv_state, x), out = act(weight . window + bias), then
 * conv_state keeps the window's last width-1 entries (read and written in place;
 * may be NULL only when width == 1). */
int ssm_conv1d_step(void* conv_state, const void* x, const float* weight, const float* bias, void* out,
                    int64_t batch, int64_t dim, int64_t width, int activation, int io_dtype,
                    hipStream_t stream);

/* Backward of ssm_conv1d_fwd for dout = dLoss/dout (fp32):
 *   dx required; dweight, dbias optional (NULL: not written).  Outputs are
 *   overwritten.  dweight and dbias are fixed-order sums of per-(batch, time
 *   segment) partials, added in lexical order, without atomics.
 *   workspace: at least ssm_conv1d_bwd_workspace_bytes() bytes, 256-byte aligned. */
size_t ssm_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                                      int io_dtype);
int ssm_conv1d_bwd(const void* x, const float* weight, const float* bias, const void* dout, void* dx,
                   float* dweight, float* dbias, void* workspace, size_t workspace_bytes, int64_t batch,
                   int64_t seqlen, int64_t dim, int64_t width, int activation, int io_dtype,
                   hipStream_t stream);

/* ssm_conv1d_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as ssm_conv1d_bwd; the weight and
 * bias partials go to a fixed scratch array inside the library instead:
 *   - SSM_CONV1D_SCRATCH_BYTES (16 MiB) per GPU, held by every GPU the library runs on
 *     until the process ends.  Sizes whose ssm_conv1d_bwd_workspace_bytes() exceeds it
 *     return SSM_ERR_SCRATCH, checked before anything is enqueued.
 *   - The array's device address is looked up (hipGetSymbolAddress) on the first call
 *     on each device; no call allocates, frees or calls an allocating routine.
 *   - Every call on one GPU uses that GPU's one array, so calls that may overlap in
 *     time on one GPU (different streams without ordering, several host threads) race
 *     and give undefined results: order them on one stream or synchronise.  Nothing
 *     needs to start at zero; every partial the reduction reads is written first. */
#define SSM_CONV1D_SCRATCH_BYTES ((size_t)16 << 20)
int ssm_conv1d_bwd_noalloc(const void* x, const float* weight, const float* bias, const void* dout,
                           void* dx, float* dweight, float* dbias, int64_t batch, int64_t seqlen,
                           int64_t dim, int64_t width, int activation, int io_dtype,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_CONV1D_H */
