/*
 * ssm_ssd.h -- C ABI of the Mamba-2 SSD chunk cumsum and its ordered backward in
 * libssmscan.so.
 *
 * The operation is the step of the Mamba-2 chunked scan (SSD) that turns raw step
 * sizes into the per-chunk decay exponents, as the pretraining_mamba2_outer page
 * deterministic_backward.py drives it through ordered_cumsum (its arguments dt, A,
 * dt_bias, dt_softplus, dt_limit, and the chunk derivatives ddA, ddt_out of shape
 * [batch, heads, chunks, width]).  With g = softplus when dt_softplus is set, else the
 * identity, and chunk c covering steps c*chunk .. c*chunk + chunk - 1:
 *
 *   forward  dt_out[b,h,c,l]    = clamp(g(dt[b, c*chunk + l, h] + dt_bias[h]), dt_min, dt_max)
 *                                 (0 for steps past the end of the sequence)
 *            dA_cumsum[b,h,c,l] = sum over l' <= l of dt_out[b,h,c,l'] * A[h]
 *   backward ddt[b,t,h]         = (ddt_out + A[h] * sum over l' >= l of ddA[b,h,c,l'])
 *                                 * mask * g'(dt + dt_bias),
 *                                 mask = 1 where g(dt + dt_bias) lies in [dt_min, dt_max]
 *                                 (bounds included), else 0
 *            dA[h]              = sum over (b, c) of sum over l of
 *                                 dt_out[b,h,c,l] * sum over l' >= l of ddA[b,h,c,l']
 *            d_dt_bias[h]       = sum over (b, c) of sum over l of ddt[b, c*chunk + l, h]
 * The page computes one partial per (batch, chunk) and adds the partials in lexical
 * (batch, chunk) order in fp32 instead of using atomics.  Here each partial is a fixed
 * tree inside one workgroup, written to the workspace, and a second kernel adds them in
 * ascending (batch, chunk) order: results are bit-identical from run to run.
 * dt_min = 0 and dt_max = +inf is no clamp with softplus (softplus > 0); without
 * softplus the lower bound 0 still clamps negative steps to 0, as the page's default
 * dt_limit = (0, inf) does.
 *
 * Layout: row-major, last index fastest; all fp32.
 *   dt, ddt                             : [batch, seqlen, heads]
 *   A, dt_bias, dA, d_dt_bias           : [heads]
 *   dA_cumsum, dt_out, ddA, ddt_out     : [batch, heads, chunks, chunk], chunks = ceil(seqlen / chunk)
 *   workspace (backward)                : the per-(batch, chunk) partials, 2 x [batch, chunks, heads]
 * Pointers are device pointers, 4-byte aligned; dt_bias may be NULL (zero), and so may
 * d_dt_bias (not written).  Outputs must not overlap inputs, each other or the
 * workspace.  The caller owns every buffer; nothing is allocated.  Work goes to
 * `stream`; the call returns without waiting.
 * Errors: an ssm_status from ssm_scan.h, every check done before any launch:
 *   SSM_ERR_NULL (a required pointer), SSM_ERR_DIM (batch, seqlen, heads or chunk < 1,
 *   heads > 2^20, 2^31 elements or more in one tensor, batch * chunks >= 2^31), SSM_ERR_ARG
 *   (dt_min < 0, dt_min > dt_max, a NaN bound), SSM_ERR_ALIGN, SSM_ERR_ALIAS,
 *   SSM_ERR_WORKSPACE (NULL, smaller than ssm_ssd_chunk_cumsum_bwd_workspace_bytes, or
 *   not 256-byte aligned), SSM_ERR_HIP.
 */
#ifndef SSM_SSD_H
#define SSM_SSD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int ssm_ssd_chunk_cumsum_fwd(const float* dt, const float* A, const float* dt_bias, float* dA_cumsum,
                             float* dt_out, int64_t batch, int64_t seqlen, int64_t heads, int64_t chunk,
                             int dt_softplus, float dt_min, float dt_max, hipStream_t stream);
size_t ssm_ssd_chunk_cumsum_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t chunk);
int ssm_ssd_chunk_cumsum_bwd(const float* ddA, const float* ddt_out, const float* dt, const float* A,
                             const float* dt_bias, float* ddt, float* dA, float* d_dt_bias, void* workspace,
                             size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t heads, int64_t chunk,
                             int dt_softplus, float dt_min, float dt_max, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SSD_H */
