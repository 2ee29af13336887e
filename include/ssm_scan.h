/*
 * ssm_scan.h -- C ABI of libssmscan.so, the gfx950 (MI355X) selective-scan library.
 *
 * The operation (Mamba selective scan, names as on the pages):
 *   Delta[b,t,d] = softplus(delta_raw[b,t,d] + dt_bias[d])      discretisation
 *   A[d,n]       = -exp(A_log[d,n])
 *   h_t[b,d,n]   = exp(Delta_t A[d,n]) h_{t-1}[b,d,n] + Delta_t B[b,t,n] x[b,t,d]
 *   s_t[b,d]     = sum_n C[b,t,n] h_t[b,d,n] + D[d] x[b,t,d]    readout from the updated state
 *   y[b,t,d]     = s_t silu(z[b,t,d])   (y = s_t when z is NULL)  optional SiLU gate
 * Passages that define it: the selective_scan_kernel and its softplus device
 * function in the POPCORNBENCH transcript FW-GLM-5-1 l2_p30 (recurrence order,
 * readout after the update, skip term D*x); mamba-rs kernels.rs, MambaKernels
 * fields (ssm_step_fwd, the one-step forward used at inference; exp_negate;
 * softplus_fwd; split_gate_silu and gating_backward, by which the SiLU gate
 * multiplies the whole SSM output; the gradient shapes of
 * ssm_reduce_d_B/_C/_D/_a_log).
 *
 * Conventions shared by every entry point
 *   Layout: contiguous row-major, last index fastest.
 *     x, delta_raw, z, y, dy, dx, ddelta_raw, dz : [batch, seqlen, d_inner]
 *     B, C                                      : [batch, seqlen, d_state]  (shared by all channels)
 *     dB, dC                                    : [batch, seqlen, d_state]  fp32
 *     A_log, dA_log                             : [d_inner, d_state]        fp32
 *     D_skip, dt_bias, dD, d_dt_bias            : [d_inner]                 fp32
 *     h0, h_final, state                        : [batch, d_inner, d_state] fp32
 *   io_dtype (ssm_dtype) is the element type of x, delta_raw, z, B, C, y (and of
 *   dy, dx, ddelta_raw, dz in the backward).  Parameters, states and all
 *   arithmetic are fp32.  bf16 results are rounded to nearest even.
 *   Pointers are device pointers (hipMalloc / torch CUDA tensors), naturally
 *   aligned for their element type.  Outputs must not overlap inputs, except
 *   `state` of ssm_scan_step, which is read and written in place.
 *   Ownership: the caller allocates and frees every buffer, including any
 *   workspace; the library allocates no device memory and keeps no pointer
 *   after a call returns.  (The one exception is the fixed scratch array of
 *   ssm_conv1d_bwd_noalloc in ssm_conv1d.h, part of the loaded code object.)
 *   Asynchrony: work is enqueued on `stream` (NULL = the default stream) and the
 *   call returns without waiting.  Faults inside a kernel surface at the
 *   caller's next synchronisation.
 *   Errors: every call returns an ssm_status.  Arguments are validated before
 *   anything is enqueued, so a call that returns a validation error has launched
 *   nothing.  A launch failure returns SSM_ERR_HIP.  No C++ exception crosses
 *   this boundary.  ssm_status_string() names a status.
 *   Determinism: for fixed sizes every output is bit-identical from run to run;
 *   sums over channels, batch and time are taken in a fixed order, with no
 *   atomics.
 *   Supported sizes: batch, seqlen, d_inner >= 1; 1 <= d_state <= 16.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,        /* a required pointer is NULL                          */
  SSM_ERR_DIM = 2,         /* a size is out of range                              */
  SSM_ERR_UNSUPPORTED = 3, /* valid request this library does not handle          */
  SSM_ERR_ALIGN = 4,       /* a pointer is not aligned to its element size        */
  SSM_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required          */
  SSM_ERR_ALIAS = 6,       /* an output overlaps an input                         */
  SSM_ERR_HIP = 7,         /* the HIP runtime reported an error at launch         */
  SSM_ERR_ARG = 8,         /* an option value is out of range                     */
  SSM_ERR_SCRATCH = 9      /* a no-allocation entry point would need more scratch
                              than the library's fixed array holds                */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* ssm_status_string(int status);

/* Forward scan over a whole sequence.
 *   Inputs : x, delta_raw, B, C (io_dtype); A_log (fp32) required.
 *            z (io_dtype) optional: NULL means no gate.
 *            D_skip, dt_bias (fp32) optional: NULL means zero.
 *            h0 (fp32) optional: NULL means a zero initial state.
 *   Outputs: y (io_dtype) required; h_final (fp32) optional (NULL: not written),
 *            the state after the last step.
 *   workspace: scratch of the time-split path (mamba-rs kernels.rs, MambaKernels
 *            ssm_parallel_fwd: the parallel-prefix forward of long sequences).  When
 *            batch * ceil(d_inner / 4) is below 1024 and seqlen is at least 1024, the
 *            sequence is cut into segments scanned in parallel and joined by a scan of
 *            their (decay, increment) pairs; ssm_scan_fwd_workspace_bytes() gives the bytes
 *            that path needs, 0 for sizes that run unsplit.  The choice depends on the
 *            sizes alone; when the size is > 0 the workspace is required (256-byte
 *            aligned, not overlapping any argument; SSM_ERR_WORKSPACE otherwise), and
 *            it is ignored when the size is 0.  Contents on entry are ignored.
 *   io_dtype: SSM_F32 or SSM_BF16.
 *   Limits: one batch element's slice, seqlen * max(d_inner, d_state) elements of
 *   io_dtype, must be below 2^31 bytes (SSM_ERR_UNSUPPORTED otherwise); d_inner
 *   <= 2^24 and seqlen <= 2^30 (SSM_ERR_DIM otherwise). */
size_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                    int64_t d_state, int io_dtype);
int ssm_scan_fwd(const void* x, const void* delta_raw, const void* z, const void* B,
                 const void* C, const float* A_log, const float* D_skip, const float* dt_bias,
                 const float* h0, void* y, float* h_final, int64_t batch, int64_t seqlen,
                 int64_t d_inner, int64_t d_state, int io_dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Single-step decode update (the scan at seqlen = 1), state updated in place.
 *   state [batch, d_inner, d_state] fp32, read and written.
 *   x, delta_raw, z (z optional) : [batch, d_inner] io_dtype.
 *   B, C                         : [batch, d_state] io_dtype.
 *   y                            : [batch, d_inner] io_dtype, written. */
int ssm_scan_step(float* state, const void* x, const void* delta_raw, const void* z,
                  const void* B, const void* C, const float* A_log, const float* D_skip,
                  const float* dt_bias, void* y, int64_t batch, int64_t d_inner,
                  int64_t d_state, int io_dtype, hipStream_t stream);

/* Backward of ssm_scan_fwd for the loss gradient dy = dLoss/dy.
 *   Inputs : the forward's inputs (same meaning, h0 optional) and dy (io_dtype).
 *   Outputs (overwritten, never accumulated):
 *     dx, ddelta_raw (io_dtype, required), dz (io_dtype, required iff z != NULL),
 *     dB, dC (fp32, required), dA_log, dD, d_dt_bias (fp32, optional: NULL means
 *     not written).  dD and d_dt_bias are the gradients as if D_skip / dt_bias
 *     were present (they are when NULL, with value zero).
 *   The gradient flowing into h_final is taken as zero and no gradient of h0 is
 *   produced (ssm_scan_bwd_ex takes the one and returns the other).
 *   workspace: required, at least ssm_scan_bwd_workspace_bytes() bytes, 256-byte
 *   aligned; its contents on entry are ignored.
 *   Reductions: dB and dC (sums over channels), dA_log, dD and d_dt_bias (sums
 *   over batch and time) are fixed-order fp32 sums of per-tile partials, without
 *   atomics, following the single-writer ordered-reduction policy of
 *   deterministic_backward.py (ordered_cumsum: partials added in lexical
 *   (batch, chunk) order) and the deterministic row partial of
 *   mamba3_preprocess_backward.slang (dt_bias_partial).
 *   Limits: as the forward, one batch element's slice, seqlen * max(d_inner, d_state)
 *   elements of io_dtype, must be below 2^31 bytes (SSM_ERR_UNSUPPORTED otherwise).
 *   io_dtype SSM_F32 or SSM_BF16: x, delta_raw, z, B, C, dy are read and dx, ddelta_raw,
 *   dz written in io_dtype (bf16 rounded to nearest even); dB, dC and the parameter
 *   gradients are fp32 in both cases, as are the state and all arithmetic. */
size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                    int64_t d_state, int io_dtype);
int ssm_scan_bwd(const void* x, const void* delta_raw, const void* z, const void* B,
                 const void* C, const float* A_log, const float* D_skip, const float* dt_bias,
                 const float* h0, const void* dy, void* dx, void* ddelta_raw, void* dz,
                 float* dB, float* dC, float* dA_log, float* dD, float* d_dt_bias,
                 void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen,
                 int64_t d_inner, int64_t d_state, int io_dtype, hipStream_t stream);

/* ---- Variants of the same path: the step-size clamp, and sequences carried across
 * segments.  The _ex entry points take the arguments of the entry points above plus
 * an options pointer; NULL (or a zero-initialised struct) gives exactly the results
 * of the plain entry points, which are the _ex calls with NULL options. */
typedef struct {
  /* Step-size clamp (mamba3_preprocess_backward.slang: dt clamp and dt mask):
   *   Delta = clamp(softplus(delta_raw + dt_bias), dt_min, dt_max),
   * and the backward passes dLoss/dDelta on to delta_raw (and dt_bias) only at steps
   * whose softplus lies inside [dt_min, dt_max], bounds included.
   * dt_min >= 0; dt_max <= 0 means no upper bound; otherwise dt_min <= dt_max.
   * A NaN bound, a negative dt_min or dt_min > dt_max > 0 gives SSM_ERR_ARG. */
  float dt_min;
  float dt_max;
  /* Backward only (NULL for the forward and the step, SSM_ERR_ARG otherwise); the
   * initial / final state gradients of a sequence carried across segments
   * (deterministic_backward.py: initial_states, dfinal_states):
   *   dh_final [batch, d_inner, d_state] fp32, read: dLoss/dh_final, the gradient that
   *            reaches the state after the last step from outside; NULL means zero.
   *   dh0      [batch, d_inner, d_state] fp32, written: dLoss/dh0; NULL: not written.
   * Both naturally aligned; dh_final must not overlap an output, dh0 nothing else. */
  const float* dh_final;
  float* dh0;
  /* Chunk states [batch, ceil(seqlen / 16), d_state, d_inner] fp32 (not allowed in the
   * step): the state entering every 16-step chunk, h_{16k-1} (h0 for k = 0), the
   * forward's states saved for reuse by the backward.  ssm_scan_fwd_ex writes them
   * (d_state 9..16 only, SSM_ERR_UNSUPPORTED otherwise); ssm_scan_bwd_ex given them
   * skips recomputing the forward states.  The backward must get the states its own
   * inputs and options produce.  ssm_scan_chunk_states_bytes() gives the size; one
   * batch element's part must stay below 2^31 bytes (SSM_ERR_UNSUPPORTED). */
  float* chunk_states;
} ssm_scan_options;

size_t ssm_scan_chunk_states_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state);

int ssm_scan_fwd_ex(const void* x, const void* delta_raw, const void* z, const void* B,
                    const void* C, const float* A_log, const float* D_skip, const float* dt_bias,
                    const float* h0, void* y, float* h_final, int64_t batch, int64_t seqlen,
                    int64_t d_inner, int64_t d_state, int io_dtype, void* workspace,
                    size_t workspace_bytes, const ssm_scan_options* options, hipStream_t stream);
int ssm_scan_step_ex(float* state, const void* x, const void* delta_raw, const void* z,
                     const void* B, const void* C, const float* A_log, const float* D_skip,
                     const float* dt_bias, void* y, int64_t batch, int64_t d_inner,
                     int64_t d_state, int io_dtype, const ssm_scan_options* options,
                     hipStream_t stream);
int ssm_scan_bwd_ex(const void* x, const void* delta_raw, const void* z, const void* B,
                    const void* C, const float* A_log, const float* D_skip, const float* dt_bias,
                    const float* h0, const void* dy, void* dx, void* ddelta_raw, void* dz,
                    float* dB, float* dC, float* dA_log, float* dD, float* d_dt_bias,
                    void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen,
                    int64_t d_inner, int64_t d_state, int io_dtype,
                    const ssm_scan_options* options, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
