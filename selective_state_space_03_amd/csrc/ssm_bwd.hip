// ssm_bwd.hip -- backward of the selective scan for gfx950 (fp32 I/O).
//
// Gradients of the loss sum(dy * y) (mamba-rs kernels.rs, MambaKernels fields, lists
// the pieces: ssm_backward_local for the per-element state, input and step-size
// contributions; ssm_reduce_d_B / _d_C into [B*T*d_state] buffers; ssm_reduce_d_D over
// d_inner; ssm_reduce_d_a_log over d_inner*d_state; softplus_bwd, silu_bwd,
// gating_backward).  With
// a_t = exp(Delta_t A), g_t = dy_t silu(z_t), and G_t = dLoss/dh_t:
//   G_t = g_t C_t + a_{t+1} G_{t+1}
//   dz_t = dy_t s_t silu'(z_t)                 dx_t = g_t D + Delta_t sum_n G_t B_t
//   dDelta_t = sum_n G_t (A a_t h_{t-1} + B_t x_t),   ddelta_raw_t = dDelta_t sigmoid(r_t)
//   dB_t = sum_d G_t Delta_t x_t   dC_t = sum_d g_t h_t   (sums over channels)
//   dA_log = A * sum_{b,t} G_t Delta_t a_t h_{t-1}, dD = sum g x, d_dt_bias = sum ddelta_raw
// The derivative of softplus is the logistic sigmoid (mamba3_preprocess_backward.slang
// writes it 1 - exp(-softplus)).
//
// Determinism (deterministic_backward.py keeps the forward as it is and fixes the
// order in which shared-parameter gradients are summed -- its ordered_cumsum adds
// per-(batch, chunk) partials batch by batch, chunk by chunk; the Slang shader writes
// a per-row dt_bias partial instead of a float atomic): there are
// no atomics.  Every sum is a fixed-order fp32 sum -- over the 64 channels of a
// tile inside one wavefront, then over tiles / batch in ascending order in a
// separate reduction kernel.
//
// Kernels, all on the caller's stream:
//   1. chunk_state : per (b, time chunk, channel) the chunk's end state from a zero
//                    start and the chunk's sum of Delta (chunks are independent);
//   2. chunk_pass  : sequential over chunks per (b, d, n): the true start state of
//                    every chunk (h0 for chunk 0);
//   3. bwd_main    : per (b, 64-channel tile), chunks in reverse order; inside a
//                    chunk the forward is recomputed from its start state with the
//                    states kept in VGPRs, then the reverse recurrence runs;
//   4. reduce_bc / reduce_params : ordered sums of the per-tile partials.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

namespace {
constexpr int kChunk = 16;  // time steps per chunk (recompute window held in VGPRs)
constexpr int kSub = 8;     // reverse steps between channel reductions of dB/dC
constexpr int kRowPad = 66; // padded LDS row (float2) for the channel reduction

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int dstate) {
  BwdLayout l;
  l.chunk = kChunk;
  l.nchunks = (seqlen + kChunk - 1) / kChunk;
  l.ngroups = (dim + 63) / 64;
  const size_t f = sizeof(float);
  size_t off = 0;
  l.off_hloc = off;     off = align256(off + (size_t)batch * l.nchunks * dim * dstate * f);
  l.off_sumdelta = off; off = align256(off + (size_t)batch * l.nchunks * dim * f);
  l.off_hstart = off;   off = align256(off + (size_t)batch * l.nchunks * dim * dstate * f);
  l.off_dbc = off;      off = align256(off + 2 * (size_t)batch * l.ngroups * seqlen * dstate * f);
  l.off_dparam = off;   off = align256(off + ((size_t)batch * dim * dstate + 2 * (size_t)batch * dim) * f);
  l.total = off;
  return l;
}

namespace {

// ---- 1. chunk end states from a zero start; lane = channel, all states per lane
template <int NS>
__global__ void __launch_bounds__(64)
chunk_state_kernel(const float* __restrict__ x, const float* __restrict__ delta_raw,
                   const float* __restrict__ Bm, const float* __restrict__ A_log,
                   const float* __restrict__ dt_bias, float* __restrict__ hloc,
                   float* __restrict__ sumdelta, int64_t L, int64_t Dm, int N, int64_t ngroups,
                   int64_t nchunks) {
  // block -> (b, chunk, group); the last chunk's end state is never needed
  const int64_t per_b = (nchunks - 1) * ngroups;
  const int64_t b = blockIdx.x / per_b;
  const int64_t rem = blockIdx.x % per_b;
  const int64_t k = rem / ngroups;
  const int64_t d = (rem % ngroups) * 64 + threadIdx.x;
  if (d >= Dm) return;  // no barriers in this kernel
  const float bias = dt_bias ? dt_bias[d] : 0.f;
  float A2[NS], h[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    A2[n] = n < N ? a2_from_alog(A_log[d * N + n]) : 0.f;
    h[n] = 0.f;
  }
  const int64_t t0 = k * kChunk;
  const int64_t t1 = (t0 + kChunk < L) ? t0 + kChunk : L;
  float sd = 0.f;
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t idx = (b * L + t) * Dm + d;
    const float delta = softplus_f(delta_raw[idx] + bias);
    const float dxv = delta * x[idx];
    sd += delta;
    const float* __restrict__ Bt = Bm + (b * L + t) * N;
#pragma unroll
    for (int n = 0; n < NS; ++n)
      if (n < N) h[n] = fmaf(exp2_hw(delta * A2[n]), h[n], dxv * Bt[n]);
  }
  const int64_t o = (b * nchunks + k) * Dm + d;
#pragma unroll
  for (int n = 0; n < NS; ++n)
    if (n < N) hloc[o * N + n] = h[n];
  sumdelta[o] = sd;
}

// ---- 2. start state of every chunk, sequential over chunks per (b, d, n)
__global__ void __launch_bounds__(256)
chunk_pass_kernel(const float* __restrict__ hloc, const float* __restrict__ sumdelta,
                  const float* __restrict__ A_log, const float* __restrict__ h0,
                  float* __restrict__ hstart, int64_t batch, int64_t Dm, int N, int64_t nchunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, d, n)
  if (i >= batch * Dm * N) return;
  const int64_t b = i / (Dm * N);
  const int64_t dn = i % (Dm * N);
  const int64_t d = dn / N;
  const float A2 = a2_from_alog(A_log[dn]);
  float h = h0 ? h0[i] : 0.f;
  for (int64_t k = 0; k < nchunks; ++k) {
    const int64_t o = (b * nchunks + k) * Dm + d;
    hstart[o * N + (dn % N)] = h;
    if (k + 1 < nchunks) h = fmaf(exp2_hw(A2 * sumdelta[o]), h, hloc[o * N + (dn % N)]);
  }
}

// ---- 3. main backward: recompute + reverse, per (b, 64-channel tile)
template <int S, int G, bool GATED>
__global__ void __launch_bounds__(64 * G)
bwd_main_kernel(const float* __restrict__ x, const float* __restrict__ delta_raw,
                const float* __restrict__ z, const float* __restrict__ Bm, const float* __restrict__ Cm,
                const float* __restrict__ A_log, const float* __restrict__ D_skip,
                const float* __restrict__ dt_bias, const float* __restrict__ dy,
                const float* __restrict__ hstart, float* __restrict__ dx, float* __restrict__ ddelta_raw,
                float* __restrict__ dz, float* __restrict__ pdB, float* __restrict__ pdC,
                float* __restrict__ pdA, float* __restrict__ pdD, float* __restrict__ pdbias,
                int64_t L, int64_t Dm, int N, int64_t ngroups, int64_t nchunks) {
  constexpr int TC = kChunk;
  constexpr int EPL = (TC + G - 1) / G;
  constexpr int NPAIR = kSub * S;      // (step, state) outputs per sub-tile and wave
  constexpr int LPP = 64 / NPAIR;      // lanes that share one output's channel sum
  static_assert(LPP >= 2 && 64 % NPAIR == 0, "sub-tile reduction layout");
  __shared__ float4 pd[TC * 64];                 // (Delta, Delta*x, g, -) per (t, channel)
  __shared__ float2 pp[TC * G * 64];             // per-wave partials: .x readout, then (P1, P2)
  __shared__ float2 scr[G][NPAIR * kRowPad];     // per-wave dB/dC channel-reduction scratch
  __shared__ float2 fin[G * 64];                 // per-wave dD / d_dt_bias partials

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.x / ngroups;
  const int64_t grp = blockIdx.x % ngroups;
  const int64_t d = grp * 64 + lane;
  const bool dvalid = d < Dm;
  const float bias = (dvalid && dt_bias) ? dt_bias[d] : 0.f;
  const float dsk = (dvalid && D_skip) ? D_skip[d] : 0.f;
  const int n0 = wave * S;
  const int nact = N - n0 < 0 ? 0 : (N - n0 > S ? S : N - n0);

  float A2[S], Av[S], Gs[S], dA[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool v = dvalid && j < nact;
    const float al = v ? A_log[d * N + n0 + j] : 0.f;
    Av[j] = v ? -expf(al) : 0.f;
    A2[j] = Av[j] * kLog2e;
    Gs[j] = 0.f;
    dA[j] = 0.f;
  }
  float dD_acc = 0.f, db_acc = 0.f;
  const int64_t row0 = b * L;

  for (int64_t k = nchunks - 1; k >= 0; --k) {
    const int64_t t0 = k * TC;
    const int tvalid = (int)((L - t0) < TC ? (L - t0) : TC);
    // ---- P: per-element values (each element once, spread over all waves)
    float ex[EPL], edelta[EPL], eg[EPL], esig[EPL], egz[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      const bool v = dvalid && t < tvalid;
      const int64_t idx = (row0 + t0 + t) * Dm + d;
      const float xv = v ? x[idx] : 0.f;
      const float r = (v ? delta_raw[idx] : 0.f) + bias;
      const float dyv = v ? dy[idx] : 0.f;
      const float delta = v ? softplus_f(r) : 0.f;
      float g = dyv, gz = 0.f;
      if (GATED) {
        const float zv = v ? z[idx] : 0.f;
        const float sz = sigmoid_f(zv);
        g = dyv * zv * sz;
        gz = dyv * sz * fmaf(zv, 1.f - sz, 1.f);
      }
      ex[i] = xv; edelta[i] = delta; eg[i] = g; esig[i] = sigmoid_f(r); egz[i] = gz;
      if (t < TC) pd[t * 64 + lane] = make_float4(delta, delta * xv, g, 0.f);
    }
    __syncthreads();
    // ---- F: recompute this wave's states over the chunk, keep h_t and a_t
    float H[TC][S], AS[TC][S], hs[S];
    {
      const float* __restrict__ hst = hstart + ((b * nchunks + k) * Dm + d) * N + n0;
#pragma unroll
      for (int j = 0; j < S; ++j) hs[j] = (dvalid && j < nact) ? hst[j] : 0.f;
      float hc[S];
#pragma unroll
      for (int j = 0; j < S; ++j) hc[j] = hs[j];
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        const int64_t tr = (t0 + t < L) ? t0 + t : L - 1;  // clamp: invalid steps have Delta = 0
        const float* __restrict__ Bt = Bm + (row0 + tr) * N + n0;
        const float* __restrict__ Ct = Cm + (row0 + tr) * N + n0;
        const float4 v = pd[t * 64 + lane];
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < S; ++j) {
          if (j < nact) {
            const float a = exp2_hw(v.x * A2[j]);
            hc[j] = fmaf(a, hc[j], v.y * Bt[j]);
            acc = fmaf(Ct[j], hc[j], acc);
            AS[t][j] = a;
          } else {
            AS[t][j] = 1.f;
          }
          H[t][j] = hc[j];
        }
        pp[(t * G + wave) * 64 + lane].x = acc;
      }
    }
    __syncthreads();
    // ---- R1: readout s_t (fixed wave order) -> dz
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      if (GATED && t < tvalid && dvalid) {
        float s = dsk * ex[i];
#pragma unroll
        for (int w = 0; w < G; ++w) s += pp[(t * G + w) * 64 + lane].x;
        dz[(row0 + t0 + t) * Dm + d] = egz[i] * s;
      }
    }
    __syncthreads();
    // ---- V: reverse recurrence over the chunk
    float2* __restrict__ sw = scr[wave];
#pragma unroll
    for (int t = TC - 1; t >= 0; --t) {
      const int64_t tr = (t0 + t < L) ? t0 + t : L - 1;
      const float* __restrict__ Bt = Bm + (row0 + tr) * N + n0;
      const float* __restrict__ Ct = Cm + (row0 + tr) * N + n0;
      const float4 v = pd[t * 64 + lane];  // Delta, Delta*x, g
      float P1 = 0.f, P2 = 0.f;
#pragma unroll
      for (int j = 0; j < S; ++j) {
        float dBp = 0.f, dCp = 0.f;
        if (j < nact) {
          const float bj = Bt[j];
          Gs[j] = fmaf(v.z, Ct[j], Gs[j]);             // dLoss/dh_t
          dCp = v.z * H[t][j];
          dBp = Gs[j] * v.y;
          P1 = fmaf(Gs[j], bj, P1);
          const float hprev = t > 0 ? H[t - 1][j] : hs[j];
          const float w = Gs[j] * (AS[t][j] * hprev);  // G a h_{t-1}
          dA[j] = fmaf(w, v.x, dA[j]);
          P2 = fmaf(w, Av[j], P2);
          Gs[j] *= AS[t][j];                            // carry to h_{t-1}
        }
        sw[((t % kSub) * S + j) * kRowPad + lane] = make_float2(dBp, dCp);
      }
      pp[(t * G + wave) * 64 + lane] = make_float2(P1, P2);
      if (t % kSub == 0) {
        // channel sums of this sub-tile: output pair p = (step, state), LPP lanes each
        // add 64/LPP channels in ascending order, then a fixed butterfly joins them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        const int p = lane / LPP, part = lane % LPP;
        float sB = 0.f, sC = 0.f;
#pragma unroll
        for (int i = 0; i < 64 / LPP; ++i) {
          const float2 q = sw[p * kRowPad + part + LPP * i];
          sB += q.x;
          sC += q.y;
        }
#pragma unroll
        for (int m = 1; m < LPP; m <<= 1) {
          sB += __shfl_xor(sB, m, LPP);
          sC += __shfl_xor(sC, m, LPP);
        }
        const int ts = t + p / S;  // absolute step inside the chunk
        const int j = p % S;
        if (part < 2 && j < nact && ts < tvalid) {
          const int64_t o = ((b * ngroups + grp) * L + t0 + ts) * N + n0 + j;
          if (part == 0) pdB[o] = sB; else pdC[o] = sC;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
    // ---- R2: per-element gradients
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      if (t < tvalid && dvalid) {
        float P1 = 0.f, P2 = 0.f;
#pragma unroll
        for (int w = 0; w < G; ++w) {
          const float2 q = pp[(t * G + w) * 64 + lane];
          P1 += q.x;
          P2 += q.y;
        }
        const int64_t idx = (row0 + t0 + t) * Dm + d;
        dx[idx] = fmaf(eg[i], dsk, edelta[i] * P1);
        const float dr = fmaf(ex[i], P1, P2) * esig[i];
        ddelta_raw[idx] = dr;
        dD_acc = fmaf(eg[i], ex[i], dD_acc);
        db_acc += dr;
      }
    }
    __syncthreads();
  }
  // ---- per-(b, d) partials: dA raw sums, and dD / d_dt_bias joined over waves in order
  if (dvalid) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j < nact) pdA[(b * Dm + d) * N + n0 + j] = dA[j];
  }
  fin[wave * 64 + lane] = make_float2(dD_acc, db_acc);
  __syncthreads();
  if (wave == 0 && dvalid) {
    float sD = 0.f, sb = 0.f;
#pragma unroll
    for (int w = 0; w < G; ++w) {
      sD += fin[w * 64 + lane].x;
      sb += fin[w * 64 + lane].y;
    }
    pdD[b * Dm + d] = sD;
    pdbias[b * Dm + d] = sb;
  }
}

// ---- 4a. dB, dC: sum of the channel-tile partials in ascending tile order
__global__ void __launch_bounds__(256)
reduce_bc_kernel(const float* __restrict__ pdB, const float* __restrict__ pdC, float* __restrict__ dB,
                 float* __restrict__ dC, int64_t batch, int64_t L, int N, int64_t ngroups) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, t, n)
  const int64_t per_b = L * N;
  if (i >= batch * per_b) return;
  const int64_t b = i / per_b, tn = i % per_b;
  float sB = 0.f, sC = 0.f;
  for (int64_t g = 0; g < ngroups; ++g) {
    const int64_t o = (b * ngroups + g) * per_b + tn;
    sB += pdB[o];
    sC += pdC[o];
  }
  dB[i] = sB;
  dC[i] = sC;
}

// ---- 4b. dA_log, dD, d_dt_bias: sums over batch in ascending order
__global__ void __launch_bounds__(256)
reduce_params_kernel(const float* __restrict__ pdA, const float* __restrict__ pdD,
                     const float* __restrict__ pdbias, const float* __restrict__ A_log,
                     float* __restrict__ dA_log, float* __restrict__ dD, float* __restrict__ d_dt_bias,
                     int64_t batch, int64_t Dm, int N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (d, n)
  if (i < Dm * N && dA_log) {
    float s = 0.f;
    for (int64_t b = 0; b < batch; ++b) s += pdA[b * Dm * N + i];
    dA_log[i] = s * -expf(A_log[i]);  // dA/dA_log = A
  }
  if (i < Dm) {
    float sD = 0.f, sb = 0.f;
    for (int64_t b = 0; b < batch; ++b) {
      sD += pdD[b * Dm + i];
      sb += pdbias[b * Dm + i];
    }
    if (dD) dD[i] = sD;
    if (d_dt_bias) d_dt_bias[i] = sb;
  }
}

template <int S, int G>
hipError_t launch_main(const BwdArgs& a, const BwdLayout& l, char* ws, hipStream_t stream) {
  float* hstart = (float*)(ws + l.off_hstart);
  float* pdB = (float*)(ws + l.off_dbc);
  float* pdC = pdB + (size_t)a.batch * l.ngroups * a.seqlen * a.dstate;
  float* pdA = (float*)(ws + l.off_dparam);
  float* pdD = pdA + (size_t)a.batch * a.dim * a.dstate;
  float* pdb = pdD + (size_t)a.batch * a.dim;
  const unsigned blocks = (unsigned)(a.batch * l.ngroups);
  if (a.z)
    hipLaunchKernelGGL((bwd_main_kernel<S, G, true>), dim3(blocks), dim3(64 * G), 0, stream, a.x,
                       a.delta_raw, a.z, a.B, a.C, a.A_log, a.D_skip, a.dt_bias, a.dy, hstart, a.dx,
                       a.ddelta_raw, a.dz, pdB, pdC, pdA, pdD, pdb, a.seqlen, a.dim, a.dstate,
                       l.ngroups, l.nchunks);
  else
    hipLaunchKernelGGL((bwd_main_kernel<S, G, false>), dim3(blocks), dim3(64 * G), 0, stream, a.x,
                       a.delta_raw, a.z, a.B, a.C, a.A_log, a.D_skip, a.dt_bias, a.dy, hstart, a.dx,
                       a.ddelta_raw, a.dz, pdB, pdC, pdA, pdD, pdb, a.seqlen, a.dim, a.dstate,
                       l.ngroups, l.nchunks);
  return hipGetLastError();
}

template <int NS>
hipError_t launch_state(const BwdArgs& a, const BwdLayout& l, char* ws, hipStream_t stream) {
  const unsigned blocks = (unsigned)(a.batch * (l.nchunks - 1) * l.ngroups);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_state_kernel<NS>), dim3(blocks), dim3(64), 0, stream, a.x, a.delta_raw, a.B,
                     a.A_log, a.dt_bias, (float*)(ws + l.off_hloc), (float*)(ws + l.off_sumdelta),
                     a.seqlen, a.dim, a.dstate, l.ngroups, l.nchunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, void* workspace, hipStream_t stream) {
  const BwdLayout l = bwd_layout(a.batch, a.seqlen, a.dim, a.dstate);
  char* ws = (char*)workspace;
  hipError_t e;
  const int ns = a.dstate <= 4 ? 4 : (a.dstate <= 8 ? 8 : 16);
  e = ns == 4 ? launch_state<4>(a, l, ws, stream)
              : (ns == 8 ? launch_state<8>(a, l, ws, stream) : launch_state<16>(a, l, ws, stream));
  if (e != hipSuccess) return e;
  {
    const int64_t n = a.batch * a.dim * a.dstate;
    hipLaunchKernelGGL(chunk_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const float*)(ws + l.off_hloc), (const float*)(ws + l.off_sumdelta), a.A_log, a.h0,
                       (float*)(ws + l.off_hstart), a.batch, a.dim, a.dstate, l.nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // four states per wave; 4, 2 or 1 wavefronts per tile for d_state <= 16, 8, 4
  e = ns == 4 ? launch_main<4, 1>(a, l, ws, stream)
              : (ns == 8 ? launch_main<4, 2>(a, l, ws, stream) : launch_main<4, 4>(a, l, ws, stream));
  if (e != hipSuccess) return e;
  {
    float* pdB = (float*)(ws + l.off_dbc);
    float* pdC = pdB + (size_t)a.batch * l.ngroups * a.seqlen * a.dstate;
    const int64_t n = a.batch * a.seqlen * a.dstate;
    hipLaunchKernelGGL(reduce_bc_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, pdB, pdC,
                       a.dB, a.dC, a.batch, a.seqlen, a.dstate, l.ngroups);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    float* pdA = (float*)(ws + l.off_dparam);
    float* pdD = pdA + (size_t)a.batch * a.dim * a.dstate;
    float* pdb = pdD + (size_t)a.batch * a.dim;
    const int64_t n = a.dim * a.dstate > a.dim ? a.dim * a.dstate : a.dim;
    hipLaunchKernelGGL(reduce_params_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, pdA, pdD,
                       pdb, a.A_log, a.dA_log, a.dD, a.d_dt_bias, a.batch, a.dim, a.dstate);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ssm
