/*
 * ssm_mamba3.h -- C ABI of the Mamba-3 projection preprocess adjoint in libssmscan.so.
 *
 * The operation is the adjoint of the per-token preprocessing that turns one row of
 * the input projection into the SSM's inputs, as printed on the
 * mamba3_preprocess_backward.slang page (oarust crate).  One projected row holds
 *   [ z (inner) | x (inner) | B (bc_rows groups x state) | C (bc_rows x state) |
 *     dd_dt (heads) | dd_a (heads) | trap (heads) | angles (rope_angles) ]
 * (width 2*inner + 2*bc_rows*state + 3*heads + rope_angles) and the gradient row has
 * the same layout:
 *   z, x, trap, angles : the incoming gradients, copied;
 *   each B and C group : RMS-norm backward, inv = 1/sqrt(mean(v^2) + epsilon),
 *                        dot = sum(g v), dv = inv g - v inv^3 dot / state;
 *   dd_dt              : (dt_grad + adt_grad * a_token) * mask * sigmoid(raw dt),
 *                        raw dt = dd_dt + dt_bias, mask = softplus(raw dt) inside
 *                        [dt_min, dt_max] (bounds included); also the row's
 *                        dt_bias partial;
 *   dd_a               : adt_grad * dt * (heavy_tail > a_floor) * -heavy_tail'(dd_a),
 *                        dt = clamp(softplus(raw dt), dt_min, dt_max),
 *                        heavy_tail(r) = 1 + r (r >= 0), 1 / (1 - r) (r < 0),
 *                        a_token = -max(heavy_tail, a_floor).
 * (sigmoid(r) is the page's 1 - exp(-softplus(r)), computed without its cancellation.)
 * The page writes a per-row dt_bias partial instead of a float atomic; d_dt_bias, if
 * asked for, is the fixed-order sum of those partials over rows (deterministic, no
 * atomics).
 *
 * Layout: row-major, last index fastest.
 *   projected, projected_grad : [rows, width]         fp32
 *   dt_bias, d_dt_bias        : [heads]               fp32
 *   z_grad, x_grad            : [rows, inner]         fp32
 *   b_grad, c_grad            : [rows, bc_rows*state] fp32 (gradients of the normalised B, C)
 *   dt_grad, adt_grad, trap_grad, dt_bias_partial : [rows, heads] fp32
 *   angle_grad                : [rows, rope_angles]   fp32
 * Pointers are device pointers, 4-byte aligned; inputs of an empty part (size 0) may be
 * NULL.  Outputs must not overlap inputs or each other.  The caller owns every buffer;
 * nothing is allocated.  Work goes to `stream`; the call returns without waiting.
 * Errors: an ssm_status from ssm_scan.h, with every check done before any launch:
 *   SSM_ERR_NULL (a required pointer), SSM_ERR_DIM (rows < 1, a negative size,
 *   bc_rows > 0 with state < 1, a row wider than 2^31 elements), SSM_ERR_ARG
 *   (epsilon < 0 or not finite, dt_min < 0, dt_min > dt_max, a NaN bound or floor),
 *   SSM_ERR_ALIGN, SSM_ERR_ALIAS, SSM_ERR_WORKSPACE, SSM_ERR_HIP.  d_dt_bias may be
 *   NULL (not written).
 * d_dt_bias is summed in fixed-order passes (64-row chunks in ascending row order; the
 * chunk sums in eight contiguous runs, each in ascending order; then the eight run sums
 * in ascending order) through a caller workspace of
 * ssm_mamba3_preprocess_bwd_workspace_bytes(rows, heads) bytes, 256-byte aligned,
 * required when d_dt_bias is given; its contents on entry are ignored.
 */
#ifndef SSM_MAMBA3_H
#define SSM_MAMBA3_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

size_t ssm_mamba3_preprocess_bwd_workspace_bytes(int64_t rows, int64_t heads);
int ssm_mamba3_preprocess_bwd(const float* projected, const float* dt_bias, const float* z_grad,
                              const float* x_grad, const float* b_grad, const float* c_grad,
                              const float* dt_grad, const float* adt_grad, const float* trap_grad,
                              const float* angle_grad, float* projected_grad, float* dt_bias_partial,
                              float* d_dt_bias, void* workspace, size_t workspace_bytes, int64_t rows,
                              int64_t inner, int64_t state, int64_t heads, int64_t rope_angles,
                              int64_t bc_rows, float epsilon, float dt_min, float dt_max, float a_floor,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_MAMBA3_H */
