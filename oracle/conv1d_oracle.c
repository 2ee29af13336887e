/*
 * conv1d_oracle.c -- plain, sequential, fp64 CPU oracle of the depthwise causal
 * conv1d (+ optional SiLU) that precedes the selective scan in a Mamba block.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU baseline use
 * it.  It shares no code, header, table or constant with the HIP library.
 *
 * What it computes (one filter of width K per channel d, zero history before t = 0):
 *   p[b,t,d]   = sum_{k<K} w[d,k] * x[b, t-(K-1)+k, d] + bias[d]     (x = 0 for t' < 0)
 *   out[b,t,d] = silu(p) when the activation is on, else p
 * Sources:
 *   - mamba-rs kernels.rs, MambaKernels conv1d fields: conv1d_step_fwd (one decode
 *     step of the depthwise conv with SiLU), conv1d_burnin_fwd / _nosave (the
 *     multi-step forward), conv1d_step_bwd and conv1d_burnin_bwd (their backward);
 *   - deterministic_backward.py, ordered_conv: the training convolution starts from
 *     reset sequences (no initial states), and the weight / bias gradients are fp32
 *     sums of per-batch partials added in batch order.
 * Decode state: [batch, dim, K-1], the K-1 most recent inputs, oldest first.  One
 * step forms the window (state, x_t), produces out_t, and keeps the window's last
 * K-1 entries.
 * Layouts (row-major, last index fastest): x, out, dout, dx : [batch, seqlen, dim];
 * w, dw : [dim, K]; bias, dbias : [dim].
 * Backward of the loss sum(dout * out):
 *   dp[b,t,d]  = dout * silu'(p) (or dout)
 *   dx[b,t,d]  = sum_{k<K} w[d,k] * dp[b, t+(K-1)-k, d]                (dp = 0 past L)
 *   dw[d,k]    = sum_{b,t} dp[b,t,d] * x[b, t-(K-1)+k, d]
 *   dbias[d]   = sum_{b,t} dp[b,t,d]
 * Returns 0 on success, -1 on bad arguments.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

static double c_sigmoid(double r) {
  if (r >= 0.0) return 1.0 / (1.0 + exp(-r));
  double e = exp(r);
  return e / (1.0 + e);
}
static double c_silu(double z) { return z * c_sigmoid(z); }
static double c_silu_grad(double z) {
  double s = c_sigmoid(z);
  return s * (1.0 + z * (1.0 - s));
}

static int args_ok(long batch, long seqlen, long dim, long width) {
  return batch >= 1 && seqlen >= 1 && dim >= 1 && width >= 1;
}

/* pre-activation p at (b, t, d) straight from the definition */
static double pre(const double *x, const double *w, const double *bias, long seqlen, long dim, long width,
                  long b, long t, long d) {
  double p = bias ? bias[d] : 0.0;
  for (long k = 0; k < width; ++k) {
    long ts = t - (width - 1) + k;
    if (ts >= 0) p += w[d * width + k] * x[(b * seqlen + ts) * dim + d];
  }
  return p;
}

int conv1d_oracle_fwd(const double *x, const double *w, const double *bias, double *out, long batch,
                      long seqlen, long dim, long width, int silu) {
  if (!x || !w || !out || !args_ok(batch, seqlen, dim, width)) return -1;
  for (long b = 0; b < batch; ++b)
    for (long t = 0; t < seqlen; ++t)
      for (long d = 0; d < dim; ++d) {
        double p = pre(x, w, bias, seqlen, dim, width, b, t, d);
        out[(b * seqlen + t) * dim + d] = silu ? c_silu(p) : p;
      }
  return 0;
}

int conv1d_oracle_step(double *state, const double *x, const double *w, const double *bias, double *out,
                       long batch, long dim, long width, int silu) {
  if (!x || !w || !out || !args_ok(batch, 1, dim, width) || (width > 1 && !state)) return -1;
  for (long b = 0; b < batch; ++b)
    for (long d = 0; d < dim; ++d) {
      double *st = state ? state + (b * dim + d) * (width - 1) : NULL;
      double xt = x[b * dim + d];
      double p = bias ? bias[d] : 0.0;
      /* window position k holds state[k] for k < K-1 and x_t at k = K-1 */
      for (long k = 0; k < width - 1; ++k) p += w[d * width + k] * st[k];
      p += w[d * width + width - 1] * xt;
      out[b * dim + d] = silu ? c_silu(p) : p;
      for (long k = 0; k + 1 < width - 1; ++k) st[k] = st[k + 1];
      if (width > 1) st[width - 2] = xt;
    }
  return 0;
}

int conv1d_oracle_bwd(const double *x, const double *w, const double *bias, const double *dout, double *dx,
                      double *dw, double *dbias, long batch, long seqlen, long dim, long width, int silu) {
  if (!x || !w || !dout || !dx || !args_ok(batch, seqlen, dim, width)) return -1;
  /* dp over the whole tensor first, then each gradient by its definition */
  size_t n = (size_t)batch * seqlen * dim;
  double *dp = (double *)malloc(n * sizeof(double));
  if (!dp) return -1;
  for (long b = 0; b < batch; ++b)
    for (long t = 0; t < seqlen; ++t)
      for (long d = 0; d < dim; ++d) {
        size_t i = (size_t)(b * seqlen + t) * dim + d;
        double g = dout[i];
        dp[i] = silu ? g * c_silu_grad(pre(x, w, bias, seqlen, dim, width, b, t, d)) : g;
      }
  for (long b = 0; b < batch; ++b)
    for (long t = 0; t < seqlen; ++t)
      for (long d = 0; d < dim; ++d) {
        double s = 0.0;
        for (long k = 0; k < width; ++k) {
          long tp = t + (width - 1) - k;
          if (tp < seqlen) s += w[d * width + k] * dp[(b * seqlen + tp) * dim + d];
        }
        dx[(b * seqlen + t) * dim + d] = s;
      }
  if (dw)
    for (long d = 0; d < dim; ++d)
      for (long k = 0; k < width; ++k) {
        double s = 0.0;
        for (long b = 0; b < batch; ++b)
          for (long t = 0; t < seqlen; ++t) {
            long ts = t - (width - 1) + k;
            if (ts >= 0) s += dp[(b * seqlen + t) * dim + d] * x[(b * seqlen + ts) * dim + d];
          }
        dw[d * width + k] = s;
      }
  if (dbias)
    for (long d = 0; d < dim; ++d) {
      double s = 0.0;
      for (long b = 0; b < batch; ++b)
        for (long t = 0; t < seqlen; ++t) s += dp[(b * seqlen + t) * dim + d];
      dbias[d] = s;
    }
  free(dp);
  return 0;
}
