/*
 * ssm_oracle.c -- plain, sequential, fp64 CPU oracle of the Mamba selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or constant with the HIP
 * library, and it does not include any of the library's headers.
 *
 * What it computes (names follow the pages' notation):
 *   Delta[b,t,d] = softplus(delta_raw[b,t,d] + dt_bias[d])
 *   A[d,n]       = -exp(A_log[d,n])
 *   h_t[b,d,n]   = exp(Delta_t * A[d,n]) * h_{t-1}[b,d,n] + Delta_t * B[b,t,n] * x[b,t,d]
 *   s_t[b,d]     = sum_n C[b,t,n] * h_t[b,d,n] + D[d] * x[b,t,d]
 *   y[b,t,d]     = s_t * silu(z[b,t,d])            (or s_t when there is no gate)
 * Sources:
 *   - the selective-scan kernel of the POPCORNBENCH transcript FW-GLM-5-1 l2_p30
 *     (its selective_scan_kernel: A_val = -exp(A_log), dA = exp(delta*A),
 *     B scaled by delta, state updated first, readout from the updated state,
 *     skip term D*x added to the readout; its softplus device function);
 *   - mamba-rs kernels.rs (MambaKernels fields): ssm_step_fwd (the one-step
 *     forward), exp_negate (A = -exp(A_log)), softplus, split_gate_silu and
 *     gating_backward (the gate multiplies the whole SSM output), and the
 *     gradient shapes of ssm_reduce_d_B/C/D/a_log;
 *   - deterministic_backward.py (ordered_cumsum): parameter-gradient sums are
 *     plain fp32-or-better sums taken in lexical (batch, chunk) order; here they
 *     are fp64 sums in (batch, time) order.
 *   - mamba3_preprocess_backward.slang (dt adjoint): d softplus / d r = 1 - exp(-softplus(r)),
 *     i.e. the logistic sigmoid of r; and its optional step-size clamp: Delta is
 *     softplus clamped to [dt_min, dt_max], and the gradient reaching delta_raw is
 *     masked to steps whose softplus lies inside the bounds (bounds included).
 *     dt_min = 0, dt_max = +inf (the default dt_limit of deterministic_backward.py's
 *     ordered_cumsum) is no clamp at all, since softplus > 0.
 *   - deterministic_backward.py (ordered_conv's initial_states / dfinal_states
 *     arguments): a sequence may start from a given state and receive a gradient on
 *     its final state; the backward then also returns the gradient of the initial
 *     state.  Here: dh_final = dLoss/dh_final enters the reverse pass as the carry
 *     beyond the last step, and dh0 = dLoss/dh0 is the carry leaving step 0.
 *
 * Layouts (row-major, last index fastest):
 *   x, delta_raw, z, y, dy, dx, ddelta_raw, dz : [batch, seqlen, dim]
 *   B, C, dB, dC                               : [batch, seqlen, dstate]
 *   A_log, dA_log                              : [dim, dstate]
 *   D, dt_bias, dD, d_dt_bias                  : [dim]
 *   h0, h_final, state                         : [batch, dim, dstate]
 * Optional inputs may be NULL: z (no gate), D (zero skip), dt_bias (zero bias),
 * h0 (zero initial state), dh_final (zero).  Optional outputs may be NULL: h_final,
 * and in the backward dz (required when z is given), dB, dC, dA_log, dD, d_dt_bias,
 * dh0.  dt_min <= dt_max are the clamp bounds (0 and +inf: no clamp).
 *
 * Threads: independent channels d are split statically across nthreads POSIX
 * threads (nthreads <= 0 means 1).  Each channel's scan is sequential in t.
 * Sums over channels (dB, dC) go into per-thread buffers that are added in
 * thread order at the end; all other outputs have a single writer.
 *
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- scalar functions (textbook definitions, fp64) ---- */

/* softplus(r) = log(1 + exp(r)), written in the overflow-free form
 * max(r, 0) + log1p(exp(-|r|)). */
double ssm_oracle_softplus(double r) {
  return (r > 0.0 ? r : 0.0) + log1p(exp(-fabs(r)));
}

/* logistic sigmoid, the derivative of softplus */
double ssm_oracle_sigmoid(double r) {
  if (r >= 0.0) return 1.0 / (1.0 + exp(-r));
  double e = exp(r);
  return e / (1.0 + e);
}

/* silu(z) = z * sigmoid(z) */
double ssm_oracle_silu(double z) { return z * ssm_oracle_sigmoid(z); }

/* d silu / dz = sigmoid(z) * (1 + z * (1 - sigmoid(z))) */
double ssm_oracle_silu_grad(double z) {
  double sg = ssm_oracle_sigmoid(z);
  return sg * (1.0 + z * (1.0 - sg));
}

/* ---- problem description shared by the thread workers ---- */

typedef struct {
  const double *x, *delta_raw, *z, *B, *C, *A_log, *D, *dt_bias, *h0, *dy, *dh_final;
  double *y, *h_final, *state;
  double *dx, *ddelta_raw, *dz, *dB, *dC, *dA_log, *dD, *d_dt_bias, *dh0;
  double dt_min, dt_max; /* clamp of Delta */
  long batch, seqlen, dim, dstate;
  long d_begin, d_end;  /* channel range owned by one worker */
  double *dB_part, *dC_part; /* per-worker [batch, seqlen, dstate] partial sums */
  int status;
} ssm_job;

/* ---- discretisation: Delta = clamp(softplus(r), dt_min, dt_max); *inside is 1 when
 * softplus(r) lies in [dt_min, dt_max] (the gradient mask), else 0 ---- */
static double discretise(const ssm_job *j, double r, double *inside) {
  const double sp = ssm_oracle_softplus(r);
  if (inside) *inside = (sp >= j->dt_min && sp <= j->dt_max) ? 1.0 : 0.0;
  return sp < j->dt_min ? j->dt_min : (sp > j->dt_max ? j->dt_max : sp);
}

/* ---- forward: one channel d of one batch element b ---- */

static void fwd_channel(const ssm_job *j, long b, long d, double *h, double *A) {
  const long L = j->seqlen, Dm = j->dim, N = j->dstate;
  for (long n = 0; n < N; ++n) {
    A[n] = -exp(j->A_log[d * N + n]);
    h[n] = j->h0 ? j->h0[(b * Dm + d) * N + n] : 0.0;
  }
  const double bias = j->dt_bias ? j->dt_bias[d] : 0.0;
  const double Dd = j->D ? j->D[d] : 0.0;
  for (long t = 0; t < L; ++t) {
    const long i = (b * L + t) * Dm + d;       /* [b, t, d] */
    const double *Bt = j->B + (b * L + t) * N; /* [b, t, :] */
    const double *Ct = j->C + (b * L + t) * N;
    const double xv = j->x[i];
    const double delta = discretise(j, j->delta_raw[i] + bias, NULL);
    double s = 0.0;
    for (long n = 0; n < N; ++n) {
      h[n] = exp(delta * A[n]) * h[n] + delta * Bt[n] * xv;
      s += Ct[n] * h[n];
    }
    s += Dd * xv;
    j->y[i] = j->z ? s * ssm_oracle_silu(j->z[i]) : s;
  }
  if (j->h_final)
    for (long n = 0; n < N; ++n) j->h_final[(b * Dm + d) * N + n] = h[n];
}

static void *fwd_worker(void *arg) {
  ssm_job *j = (ssm_job *)arg;
  double *h = malloc(sizeof(double) * j->dstate), *A = malloc(sizeof(double) * j->dstate);
  if (!h || !A) { free(h); free(A); j->status = -2; return NULL; }
  for (long d = j->d_begin; d < j->d_end; ++d)
    for (long b = 0; b < j->batch; ++b) fwd_channel(j, b, d, h, A);
  free(h); free(A);
  j->status = 0;
  return NULL;
}

/* ---- single-step decode update (written separately from the scan on purpose) ---- */

static void step_channel(const ssm_job *j, long b, long d) {
  const long Dm = j->dim, N = j->dstate;
  const long i = b * Dm + d;                   /* [b, d] */
  double *st = j->state + (b * Dm + d) * N;    /* [b, d, :] */
  const double *Bb = j->B + b * N, *Cb = j->C + b * N;
  const double xv = j->x[i];
  const double delta = discretise(j, j->delta_raw[i] + (j->dt_bias ? j->dt_bias[d] : 0.0), NULL);
  double s = 0.0;
  for (long n = 0; n < N; ++n) {
    const double A = -exp(j->A_log[d * N + n]);
    st[n] = exp(delta * A) * st[n] + delta * Bb[n] * xv;
    s += Cb[n] * st[n];
  }
  s += (j->D ? j->D[d] : 0.0) * xv;
  j->y[i] = j->z ? s * ssm_oracle_silu(j->z[i]) : s;
}

static void *step_worker(void *arg) {
  ssm_job *j = (ssm_job *)arg;
  for (long d = j->d_begin; d < j->d_end; ++d)
    for (long b = 0; b < j->batch; ++b) step_channel(j, b, d);
  j->status = 0;
  return NULL;
}

/* ---- backward: reverse-mode derivative of the forward above ----
 * Per channel: a forward pass keeps every state h_t (t = -1 .. L-1) and the
 * pre-gate output s_t; the reverse pass walks t = L-1 .. 0 carrying
 * G[n] = dLoss/dh_t[n].  With a_t = exp(Delta_t A):
 *   dLoss/ds_t        = g_t = dy_t * silu(z_t)            (dy_t without a gate)
 *   dz_t              = dy_t * s_t * silu'(z_t)
 *   G_t               = g_t C_t + a_{t+1} G_{t+1}
 *   dC[b,t,n]        += g_t h_t[n]                        (summed over d)
 *   dB[b,t,n]        += G_t[n] Delta_t x_t                (summed over d)
 *   dx_t              = g_t D + Delta_t sum_n G_t[n] B_t[n]
 *   dDelta_t          = sum_n G_t[n] (A[n] a_t[n] h_{t-1}[n] + B_t[n] x_t)
 *   ddelta_raw_t      = dDelta_t * mask_t * sigmoid(delta_raw_t + dt_bias)
 *                       (mask_t = 1 when softplus lies inside the clamp bounds, else 0)
 *   dA[n]            += G_t[n] Delta_t a_t[n] h_{t-1}[n];  dA_log = dA * A  (dA/dA_log = A)
 *   dD               += g_t x_t;   d_dt_bias += ddelta_raw_t
 * The carry starts at G = dh_final (zero when absent); after step 0 it is a_0 G_0 =
 * dLoss/dh0, written to dh0.
 */
static int bwd_channel(ssm_job *j, long b, long d, double *hs, double *s_pre, double *A,
                       double *G, double *dA_acc) {
  const long L = j->seqlen, Dm = j->dim, N = j->dstate;
  for (long n = 0; n < N; ++n) {
    A[n] = -exp(j->A_log[d * N + n]);
    hs[n] = j->h0 ? j->h0[(b * Dm + d) * N + n] : 0.0; /* hs row 0 holds h_{-1} */
  }
  const double bias = j->dt_bias ? j->dt_bias[d] : 0.0;
  const double Dd = j->D ? j->D[d] : 0.0;
  /* forward, keeping states: hs[(t+1)*N + n] = h_t[n] */
  for (long t = 0; t < L; ++t) {
    const long i = (b * L + t) * Dm + d;
    const double *Bt = j->B + (b * L + t) * N, *Ct = j->C + (b * L + t) * N;
    const double xv = j->x[i];
    const double delta = discretise(j, j->delta_raw[i] + bias, NULL);
    double s = 0.0;
    for (long n = 0; n < N; ++n) {
      const double hn = exp(delta * A[n]) * hs[t * N + n] + delta * Bt[n] * xv;
      hs[(t + 1) * N + n] = hn;
      s += Ct[n] * hn;
    }
    s_pre[t] = s + Dd * xv;
  }
  /* reverse */
  for (long n = 0; n < N; ++n) G[n] = j->dh_final ? j->dh_final[(b * Dm + d) * N + n] : 0.0;
  double dD_acc = 0.0, dbias_acc = 0.0;
  for (long t = L - 1; t >= 0; --t) {
    const long i = (b * L + t) * Dm + d;
    const long bt = (b * L + t) * N;
    const double *Bt = j->B + bt, *Ct = j->C + bt;
    const double xv = j->x[i];
    const double r = j->delta_raw[i] + bias;
    double inside;
    const double delta = discretise(j, r, &inside);
    const double dyv = j->dy[i];
    double g;
    if (j->z) {
      const double zv = j->z[i];
      g = dyv * ssm_oracle_silu(zv);
      j->dz[i] = dyv * s_pre[t] * ssm_oracle_silu_grad(zv);
    } else {
      g = dyv;
    }
    dD_acc += g * xv;
    double dxacc = 0.0, ddelta = 0.0;
    for (long n = 0; n < N; ++n) {
      const double h_prev = hs[t * N + n], h_cur = hs[(t + 1) * N + n];
      const double a = exp(delta * A[n]);
      G[n] += g * Ct[n]; /* now dLoss/dh_t[n] */
      if (j->dC_part) j->dC_part[bt + n] += g * h_cur;
      if (j->dB_part) j->dB_part[bt + n] += G[n] * delta * xv;
      dA_acc[n] += G[n] * delta * a * h_prev;
      ddelta += G[n] * (A[n] * a * h_prev + Bt[n] * xv);
      dxacc += G[n] * delta * Bt[n];
      G[n] *= a; /* contribution to dLoss/dh_{t-1}[n] through h_t */
    }
    j->dx[i] = g * Dd + dxacc;
    const double dr = ddelta * inside * ssm_oracle_sigmoid(r);
    j->ddelta_raw[i] = dr;
    dbias_acc += dr;
  }
  if (j->dD) j->dD[d] += dD_acc;
  if (j->d_dt_bias) j->d_dt_bias[d] += dbias_acc;
  if (j->dh0)
    for (long n = 0; n < N; ++n) j->dh0[(b * Dm + d) * N + n] = G[n];
  return 0;
}

static void *bwd_worker(void *arg) {
  ssm_job *j = (ssm_job *)arg;
  const long L = j->seqlen, N = j->dstate;
  double *hs = malloc(sizeof(double) * (size_t)(L + 1) * N);
  double *s_pre = malloc(sizeof(double) * (size_t)L);
  double *A = malloc(sizeof(double) * N), *G = malloc(sizeof(double) * N);
  double *dA_acc = malloc(sizeof(double) * N);
  if (!hs || !s_pre || !A || !G || !dA_acc) {
    free(hs); free(s_pre); free(A); free(G); free(dA_acc);
    j->status = -2;
    return NULL;
  }
  for (long d = j->d_begin; d < j->d_end; ++d) {
    for (long n = 0; n < N; ++n) dA_acc[n] = 0.0;
    if (j->dD) j->dD[d] = 0.0;
    if (j->d_dt_bias) j->d_dt_bias[d] = 0.0;
    for (long b = 0; b < j->batch; ++b) bwd_channel(j, b, d, hs, s_pre, A, G, dA_acc);
    if (j->dA_log)
      for (long n = 0; n < N; ++n) j->dA_log[d * N + n] = dA_acc[n] * (-exp(j->A_log[d * N + n]));
  }
  free(hs); free(s_pre); free(A); free(G); free(dA_acc);
  j->status = 0;
  return NULL;
}

/* ---- thread driver ---- */

static int run_split(ssm_job *proto, long dim, int nthreads, void *(*fn)(void *)) {
  if (nthreads <= 0) nthreads = 1;
  if (nthreads > dim) nthreads = (int)dim;
  if (nthreads < 1) nthreads = 1;
  ssm_job *jobs = calloc((size_t)nthreads, sizeof(ssm_job));
  pthread_t *tids = calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !tids) { free(jobs); free(tids); return -2; }
  int rc = 0;
  for (int k = 0; k < nthreads; ++k) {
    jobs[k] = *proto;
    jobs[k].d_begin = dim * k / nthreads;
    jobs[k].d_end = dim * (k + 1) / nthreads;
    jobs[k].status = -2;
  }
  int started = 0;
  for (int k = 1; k < nthreads; ++k) {
    if (pthread_create(&tids[k], NULL, fn, &jobs[k]) != 0) break;
    started = k;
  }
  fn(&jobs[0]);
  for (int k = 1; k <= started; ++k) pthread_join(tids[k], NULL);
  for (int k = started + 1; k < nthreads; ++k) fn(&jobs[k]); /* threads that failed to start */
  for (int k = 0; k < nthreads; ++k)
    if (jobs[k].status != 0) rc = jobs[k].status;
  free(jobs); free(tids);
  return rc;
}

static int dims_ok(long batch, long seqlen, long dim, long dstate) {
  return batch > 0 && seqlen > 0 && dim > 0 && dstate > 0;
}

static int clamp_ok(double dt_min, double dt_max) {
  return dt_min >= 0.0 && dt_min <= dt_max; /* false for NaN */
}

int ssm_oracle_fwd(const double *x, const double *delta_raw, const double *z, const double *B,
                   const double *C, const double *A_log, const double *D, const double *dt_bias,
                   const double *h0, double *y, double *h_final, long batch, long seqlen, long dim,
                   long dstate, double dt_min, double dt_max, int nthreads) {
  if (!x || !delta_raw || !B || !C || !A_log || !y) return -1;
  if (!dims_ok(batch, seqlen, dim, dstate) || !clamp_ok(dt_min, dt_max)) return -1;
  ssm_job j;
  memset(&j, 0, sizeof(j));
  j.x = x; j.delta_raw = delta_raw; j.z = z; j.B = B; j.C = C; j.A_log = A_log; j.D = D;
  j.dt_bias = dt_bias; j.h0 = h0; j.y = y; j.h_final = h_final;
  j.batch = batch; j.seqlen = seqlen; j.dim = dim; j.dstate = dstate;
  j.dt_min = dt_min; j.dt_max = dt_max;
  return run_split(&j, dim, nthreads, fwd_worker);
}

int ssm_oracle_step(double *state, const double *x, const double *delta_raw, const double *z,
                    const double *B, const double *C, const double *A_log, const double *D,
                    const double *dt_bias, double *y, long batch, long dim, long dstate,
                    double dt_min, double dt_max, int nthreads) {
  if (!state || !x || !delta_raw || !B || !C || !A_log || !y) return -1;
  if (!dims_ok(batch, 1, dim, dstate) || !clamp_ok(dt_min, dt_max)) return -1;
  ssm_job j;
  memset(&j, 0, sizeof(j));
  j.state = state; j.x = x; j.delta_raw = delta_raw; j.z = z; j.B = B; j.C = C;
  j.A_log = A_log; j.D = D; j.dt_bias = dt_bias; j.y = y;
  j.batch = batch; j.seqlen = 1; j.dim = dim; j.dstate = dstate;
  j.dt_min = dt_min; j.dt_max = dt_max;
  return run_split(&j, dim, nthreads, step_worker);
}

int ssm_oracle_bwd(const double *x, const double *delta_raw, const double *z, const double *B,
                   const double *C, const double *A_log, const double *D, const double *dt_bias,
                   const double *h0, const double *dy, const double *dh_final, double *dx,
                   double *ddelta_raw, double *dz, double *dB, double *dC, double *dA_log,
                   double *dD, double *d_dt_bias, double *dh0, long batch, long seqlen, long dim,
                   long dstate, double dt_min, double dt_max, int nthreads) {
  if (!x || !delta_raw || !B || !C || !A_log || !dy || !dx || !ddelta_raw) return -1;
  if (z && !dz) return -1;
  if (!dims_ok(batch, seqlen, dim, dstate) || !clamp_ok(dt_min, dt_max)) return -1;
  if (nthreads <= 0) nthreads = 1;
  if (nthreads > dim) nthreads = (int)dim;
  const size_t S = (size_t)batch * seqlen * dstate;
  double *parts = NULL;
  if (dB || dC) {
    parts = calloc((size_t)nthreads * 2 * S, sizeof(double));
    if (!parts) return -2;
  }
  ssm_job *jobs = calloc((size_t)nthreads, sizeof(ssm_job));
  pthread_t *tids = calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !tids) { free(parts); free(jobs); free(tids); return -2; }
  for (int k = 0; k < nthreads; ++k) {
    ssm_job *j = &jobs[k];
    j->x = x; j->delta_raw = delta_raw; j->z = z; j->B = B; j->C = C; j->A_log = A_log;
    j->D = D; j->dt_bias = dt_bias; j->h0 = h0; j->dy = dy; j->dh_final = dh_final;
    j->dx = dx; j->ddelta_raw = ddelta_raw; j->dz = dz; j->dA_log = dA_log; j->dD = dD;
    j->d_dt_bias = d_dt_bias; j->dh0 = dh0;
    j->dt_min = dt_min; j->dt_max = dt_max;
    j->batch = batch; j->seqlen = seqlen; j->dim = dim; j->dstate = dstate;
    j->d_begin = dim * k / nthreads;
    j->d_end = dim * (k + 1) / nthreads;
    j->dB_part = parts ? parts + (size_t)k * 2 * S : NULL;
    j->dC_part = parts ? parts + (size_t)k * 2 * S + S : NULL;
    j->status = -2;
  }
  int started = 0;
  for (int k = 1; k < nthreads; ++k) {
    if (pthread_create(&tids[k], NULL, bwd_worker, &jobs[k]) != 0) break;
    started = k;
  }
  bwd_worker(&jobs[0]);
  for (int k = 1; k <= started; ++k) pthread_join(tids[k], NULL);
  for (int k = started + 1; k < nthreads; ++k) bwd_worker(&jobs[k]);
  int rc = 0;
  for (int k = 0; k < nthreads; ++k)
    if (jobs[k].status != 0) rc = jobs[k].status;
  /* channel sums, added in thread (= ascending channel block) order */
  if (rc == 0 && parts) {
    for (size_t e = 0; e < S; ++e) {
      double sb = 0.0, sc = 0.0;
      for (int k = 0; k < nthreads; ++k) {
        sb += parts[(size_t)k * 2 * S + e];
        sc += parts[(size_t)k * 2 * S + S + e];
      }
      if (dB) dB[e] = sb;
      if (dC) dC[e] = sc;
    }
  }
  free(parts); free(jobs); free(tids);
  return rc;
}
