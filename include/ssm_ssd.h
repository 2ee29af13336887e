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
/*
 * ssm_ssd_chunk_scan_fwd -- the Mamba-2 SSD scan forward over chunks, fed by the chunk
 * cumsum above.  The layer whose chunked kernels deterministic_backward.py names
 * (ssd_chunk_state, ssd_state_passing, ssd_chunk_scan) is the selective recurrence
 * with one scalar decay rate A per head; per (batch b, head h) the state is a
 * [headdim, d_state] matrix:
 *   state_t = exp(dt_t A[h]) state_{t-1} + dt_t outer(x[b,t,h,:], B[b,t,:])
 *   y[b,t,h,:] = state_t C[b,t,:] + D[h] x[b,t,h,:]
 * with dt_t the clamped step dt_out and A[h] entering only through dA_cumsum (both as
 * ssm_ssd_chunk_cumsum_fwd writes them).  B and C form one group shared by every head.
 * Inside a chunk of W steps, with cs = dA_cumsum and dt = dt_out of the chunk:
 *   y_i   = exp(cs_i) C_i state_in + sum over s <= i of (C_i . B_s) exp(cs_i - cs_s) dt_s x_s
 *   state_out = exp(cs_{W-1}) state_in + sum over s of exp(cs_{W-1} - cs_s) dt_s outer(x_s, B_s)
 * which the kernel evaluates as matrix products on the matrix cores, carrying the
 * state from chunk to chunk.  Equal to the recurrence up to rounding.
 *
 * Layout: row-major, last index fastest; all fp32.
 *   x, y                  : [batch, seqlen, heads, headdim]
 *   dt_out, dA_cumsum     : [batch, heads, chunks, chunk], chunks = ceil(seqlen / chunk)
 *                           (steps past the sequence end: dt_out 0, dA_cumsum flat)
 *   B, C                  : [batch, seqlen, d_state]
 *   D                     : [heads], may be NULL (no skip term)
 *   h0, h_final           : [batch, heads, headdim, d_state], may be NULL (zero / not written)
 *   block_states          : [batch, heads, ceil(seqlen / 64), headdim, d_state], may be NULL:
 *                           the state entering every 64-step block (what the backward
 *                           below reads instead of recomputing it)
 * Supported: headdim 64, d_state 64 or 128, chunk a multiple of 64 (SSM_ERR_UNSUPPORTED
 * otherwise); a chunk is walked in blocks of 64 steps.  Inputs are expected finite: the
 * in-block products are dense matrix products, so a NaN or Inf in a 64-step block can
 * reach the outputs of every step of that block (and, through the state, later ones).
 * workspace             : ssm_ssd_chunk_scan_fwd_workspace_bytes(batch, seqlen, d_state)
 *                           bytes, 256-byte aligned, contents on entry ignored: the
 *                           products C_i.B_s of every 64-step block, [batch, blocks, 64,
 *                           64] fp32, computed once and shared by all heads
 * Pointers are device pointers, 4-byte aligned.  Outputs must not overlap inputs or
 * each other.  Nothing is allocated; work goes to `stream`.
 * Errors: SSM_ERR_NULL, SSM_ERR_DIM (a size < 1, 2^31 elements or more in one tensor,
 * batch * heads >= 2^31), SSM_ERR_UNSUPPORTED, SSM_ERR_ALIGN, SSM_ERR_ALIAS,
 * SSM_ERR_WORKSPACE (NULL, smaller than the size above or misaligned), SSM_ERR_HIP.
 */
/*
 * ssm_ssd_chunk_scan_bwd -- the gradients of ssm_ssd_chunk_scan_fwd for the loss
 * sum(dy * y) + sum(dh_final * h_final), by the reverse recurrence of the adjoint
 * state G = dLoss/dstate (G_{t-1} = exp(dt_t A) G_t + outer(dy_{t-1}, C_{t-1})), over
 * the same chunks on the matrix cores.  It reads the entering state of every chunk
 * from the forward's block_states instead of recomputing it.  Outputs:
 *   dx                    : [batch, seqlen, heads, headdim]
 *   ddA_cumsum, ddt_out   : [batch, heads, chunks, chunk], the gradients of dA_cumsum and
 *                           dt_out; ssm_ssd_chunk_cumsum_bwd turns them into the
 *                           gradients of dt, A and dt_bias
 *   dB, dC                : [batch, seqlen, d_state], summed over the heads in a fixed
 *                           order inside the workgroup of each (batch, chunk) (one writer
 *                           each, no atomics)
 *   dD                    : [heads], summed over (batch, chunk) in ascending order (may be NULL)
 *   dh0                   : [batch, heads, headdim, d_state], dLoss/dh0 (may be NULL)
 * dh_final may be NULL (zero).  D may be NULL (no skip term; dD is then still the
 * gradient of a skip weight).  block_states is required.  The workspace holds the
 * state adjoint G of every (batch, head, chunk) ([headdim, d_state] fp32 each), dD per
 * (batch, chunk, head), and, when there are at most 128 (batch, chunk) pairs and the
 * heads of a chunk are split over several workgroups, each group's dB and dC:
 * ssm_ssd_chunk_scan_bwd_workspace_bytes, 256-byte aligned, contents on entry ignored.  Supported: headdim 64, d_state 64 or
 * 128, chunk 64 (SSM_ERR_UNSUPPORTED otherwise).  Results are bit-identical from run
 * to run.  Errors as for the forward, plus SSM_ERR_WORKSPACE.
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

size_t ssm_ssd_chunk_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dstate);
int ssm_ssd_chunk_scan_fwd(const float* x, const float* dt_out, const float* dA_cumsum, const float* B,
                           const float* C, const float* D, const float* h0, float* y, float* h_final,
                           float* block_states, void* workspace, size_t workspace_bytes, int64_t batch,
                           int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate, int64_t chunk,
                           hipStream_t stream);

size_t ssm_ssd_chunk_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t dstate);
int ssm_ssd_chunk_scan_bwd(const float* x, const float* dt_out, const float* dA_cumsum, const float* B,
                           const float* C, const float* D, const float* dy, const float* block_states,
                           const float* dh_final, float* dx, float* ddA_cumsum, float* ddt_out, float* dB,
                           float* dC, float* dD, float* dh0, void* workspace, size_t workspace_bytes, int64_t batch,
                           int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate, int64_t chunk,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SSD_H */
