// ssm_bwd.hip -- backward of the selective scan for gfx950 (fp32 or bf16 I/O; state,
// arithmetic and dB, dC and the parameter gradients in fp32).
//
// Gradients of the loss sum(dy * y) (mamba-rs kernels.rs, MambaKernels fields, lists
// the pieces: ssm_backward_local for the per-element state, input and step-size
// contributions; ssm_reduce_d_B / _d_C into [B*T*d_state] buffers; ssm_reduce_d_D over
// d_inner; ssm_reduce_d_a_log over d_inner*d_state; softplus_bwd, silu_bwd,
// gating_backward).  With a_t = exp(Delta_t A), u_t = Delta_t x_t, g_t = dy_t silu(z_t)
// and G_t = dLoss/dh_t:
//   G_t = g_t C_t + a_{t+1} G_{t+1}
//   dz_t = dy_t s_t silu'(z_t)                 dx_t = g_t D + Delta_t sum_n G_t B_t
//   dDelta_t = sum_n G_t (A a_t h_{t-1} + B_t x_t),   ddelta_raw_t = dDelta_t sigmoid(r_t)
//   dB_t = sum_d G_t u_t   dC_t = sum_d g_t h_t   (sums over channels)
//   dA_log = A * sum_{b,t} G_t Delta_t a_t h_{t-1}, dD = sum g x, d_dt_bias = sum ddelta_raw
// The derivative of softplus is the logistic sigmoid (mamba3_preprocess_backward.slang
// writes it 1 - exp(-softplus)).
//
// Determinism (deterministic_backward.py keeps the forward as it is and fixes the
// order in which shared-parameter gradients are summed -- its ordered_cumsum adds
// per-(batch, chunk) partials batch by batch, chunk by chunk; the Slang shader writes
// a per-row dt_bias partial instead of a float atomic): there are no atomics.  Every
// sum is a fixed-order fp32 sum -- over the 64 channels of a tile inside one
// wavefront, over the wavefronts of a workgroup in wave order, then over tiles /
// (batch, segment) in ascending order in a separate reduction kernel.
//
// Parallel structure.  Both recurrences are linear, so time is cut into segments of
// segc chunks of kChunk steps that are processed independently; what crosses a
// segment boundary is a state (forward) and an adjoint carry (reverse), each an
// affine function of its value at the other end of the segment, with decay
// exp(A * sum of Delta over the segment):
//   1. chunk_rel : per (b, 64-channel tile, segment), forward from a zero state:
//                  the state at every chunk start relative to the segment start, the
//                  sum of Delta up to it, and the segment's end state (skipped when the
//                  forward saved the true chunk start states);
//   2. seg_adj   : per (b, tile, segment), the reverse recurrence from a zero carry:
//                  the carry leaving the segment's first step, and the segment's Delta sum;
//   3. seg_pass  : per (b, d, n), sequential over segments: the true state entering
//                  every segment (h0 first) and the true carry entering it from the
//                  right;
//   4. bwd_main  : per (b, tile, segment), chunks in reverse order: the chunk's start
//                  state from 1 and 3, its forward recomputed into VGPRs, then the
//                  reverse recurrence and every gradient;
//   5. reduce_bc / reduce_params : ordered sums of the per-tile partials.
// Work layout (as in the forward): lane = channel, the G wavefronts of a workgroup
// split the state axis (S states per wave), per-element work is done once per
// (t, channel) and shared through LDS.  B and C of a chunk are staged in LDS too and
// read with same-address (broadcast) loads: scalar loads inside the step loops would
// share the LDS wait counter and complete out of order, forcing a full wait per step.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

namespace {
constexpr int kChunk = 16;  // time steps per chunk (recompute window held in VGPRs)
constexpr int kSub = 4;     // reverse steps between channel reductions of dB/dC
constexpr int kS = 2;       // states per wavefront

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// DPP lane permutations inside rows of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sums of 16 values over the 64 lanes of a wavefront (a transpose-reduce): every
// stage pairs each lane with one in the other half of a lane group, each lane keeps
// one half of its values and adds the partner's copy of that half.  Lanes 32-63 /
// 0-31 and odd / even 16-lane rows are exchanged by the gfx950 permlane swaps, the
// 8- and 4-lane halves of a row by DPP mirrors, the last two quad steps are plain
// DPP butterflies.  Lane i ends with the sum of value (i >> 2) & 15; the tree is
// fixed, so the result is deterministic.
__device__ __forceinline__ float transpose_reduce16(float (&v)[16], int lane) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {  // lanes 0-31 keep v[k], lanes 32-63 keep v[k + 8]
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 8]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // even rows keep v[k], odd rows keep v[k + 4]
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 4]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool h3 = (lane & 8) != 0, h2 = (lane & 4) != 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // row halves (lane 15 - i is the partner): keep v[k] / v[k + 2]
    const float keep = h3 ? v[k + 2] : v[k], send = h3 ? v[k] : v[k + 2];
    v[k] = keep + dpp<kDppRowMirror>(send);
  }
  {  // quarters of a row (lane 7 - i within 8): keep v[0] / v[1]
    const float keep = h2 ? v[1] : v[0], send = h2 ? v[0] : v[1];
    v[0] = keep + dpp<kDppRowHalfMirror>(send);
  }
  v[0] += dpp<kDppQuadXor2>(v[0]);
  v[0] += dpp<kDppQuadXor1>(v[0]);
  return v[0];
}
int waves_for(int dstate) { return dstate <= 2 ? 1 : (dstate <= 4 ? 2 : (dstate <= 8 ? 4 : 8)); }
}  // namespace

BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int dstate) {
  BwdLayout l;
  l.fused = batch * ((dim + 3) / 4) >= 1024 || seqlen < 1024;
  if (l.fused) {
    // chunk states, then per-workgroup dB/dC partials, then the per-batch-element
    // parameter partials (dA [B, N, D], dD [B, D], d_dt_bias [B, D])
    const size_t f = sizeof(float), N = (size_t)dstate;
    l.chunk = kStateChunk;
    l.nchunks = (seqlen + kStateChunk - 1) / kStateChunk;
    l.ngroups = bwd_fused_groups(dim);
    l.segc = l.nchunks;
    l.nseg = 1;
    size_t off = 0;
    l.off_cs = off;     off = align256(off + (size_t)batch * l.nchunks * N * dim * f);
    l.off_dbc = off;    off = align256(off + 2 * (size_t)batch * l.ngroups * seqlen * N * f);
    l.off_dparam = off; off = align256(off + ((size_t)batch * dim * N + 2 * (size_t)batch * dim) * f);
    l.off_hrel = l.off_cumd = l.off_hseg = l.off_sdseg = l.off_gseg = l.off_hin = l.off_gin = 0;
    l.total = off;
    return l;
  }
  l.off_cs = 0;
  l.chunk = kChunk;
  l.nchunks = (seqlen + kChunk - 1) / kChunk;
  l.ngroups = (dim + 63) / 64;
  // segments: enough (batch, tile, segment) workgroups to fill the chip several times
  // over, but at least 4 chunks per segment
  const int64_t want = (2048 + batch * l.ngroups - 1) / (batch * l.ngroups);
  int64_t segc = (l.nchunks + want - 1) / want;
  if (segc < 4) segc = 4;
  if (segc > l.nchunks) segc = l.nchunks;
  l.segc = segc;
  l.nseg = (l.nchunks + segc - 1) / segc;
  const size_t f = sizeof(float);
  const size_t N = (size_t)dstate;
  size_t off = 0;
  l.off_hrel = off;   off = align256(off + (size_t)batch * l.nchunks * dim * N * f);
  l.off_cumd = off;   off = align256(off + (size_t)batch * l.nchunks * dim * f);
  l.off_hseg = off;   off = align256(off + (size_t)batch * l.nseg * dim * N * f);
  l.off_sdseg = off;  off = align256(off + (size_t)batch * l.nseg * dim * f);
  l.off_gseg = off;   off = align256(off + (size_t)batch * l.nseg * dim * N * f);
  l.off_hin = off;    off = align256(off + (size_t)batch * l.nseg * dim * N * f);
  l.off_gin = off;    off = align256(off + (size_t)batch * l.nseg * dim * N * f);
  l.off_dbc = off;    off = align256(off + 2 * (size_t)batch * l.ngroups * seqlen * N * f);
  l.off_dparam = off; off = align256(off + ((size_t)batch * l.nseg * dim * N + 2 * (size_t)batch * l.nseg * dim) * f);
  l.total = off;
  return l;
}

namespace {

// Common per-lane set-up: channel, states of this wave, and the segment's chunks.
struct Lane {
  int lane, wave;
  int64_t b, grp, seg, d;
  bool dvalid;
  int n0, nact;
  int64_t c_begin, c_end;
};
template <int S>
__device__ __forceinline__ Lane lane_setup(int64_t ngroups, int64_t nseg, int64_t segc, int64_t nchunks, int N) {
  Lane q;
  q.lane = threadIdx.x & 63;
  q.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // block -> (b, segment, group): the groups of one segment are neighbours
  q.grp = blockIdx.x % ngroups;
  const int64_t bs = blockIdx.x / ngroups;
  q.seg = bs % nseg;
  q.b = bs / nseg;
  q.d = q.grp * 64 + q.lane;
  q.n0 = q.wave * S;
  q.nact = N - q.n0 < 0 ? 0 : (N - q.n0 > S ? S : N - q.n0);
  q.c_begin = q.seg * segc;
  q.c_end = q.c_begin + segc < nchunks ? q.c_begin + segc : nchunks;
  q.dvalid = false;  // set by the caller (needs Dm)
  return q;
}

// ---- 1. forward from a zero state per segment: chunk-start states relative to the
// segment start, Delta sums, and the segment's end state.  One barrier per chunk:
// the prep of chunk c+1 goes to the other half of double-buffered LDS while chunk c
// is scanned from registers.
template <typename T, int S, int G>
__global__ void __launch_bounds__(64 * G)
chunk_rel_kernel(const T* __restrict__ x, const T* __restrict__ delta_raw,
                 const T* __restrict__ Bm, const float* __restrict__ A_log,
                 const float* __restrict__ dt_bias, float* __restrict__ hrel, float* __restrict__ cumd,
                 float* __restrict__ hseg, int64_t L, int64_t Dm, int N,
                 int64_t ngroups, int64_t nchunks, int64_t segc, int64_t nseg, float dt_lo, float dt_hi) {
  constexpr int TC = kChunk;
  constexpr int EPL = (TC + G - 1) / G;
  __shared__ float2 pd[2][TC * 64];  // (Delta, Delta*x) per (t, channel)
  __shared__ float bs[2][TC * 16];   // B per (t, state), zero beyond d_state
  Lane q = lane_setup<S>(ngroups, nseg, segc, nchunks, N);
  q.dvalid = q.d < Dm;
  const float bias = (q.dvalid && dt_bias) ? dt_bias[q.d] : 0.f;
  float A2[S], h[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    A2[j] = (q.dvalid && j < q.nact) ? a2_from_alog(A_log[q.d * N + q.n0 + j]) : 0.f;
    h[j] = 0.f;
  }
  float sd = 0.f;
  const int64_t row0 = q.b * L;
  // this wave's rows of a chunk (x, delta_raw, B), loaded one chunk ahead of the prep
  uint32_t lx[EPL], lr[EPL], lb[EPL];  // raw element bits
  auto load = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * TC;
    const int tvalid = (int)(L - t0 < TC ? L - t0 : TC);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = q.wave + G * i;
      const bool v = q.dvalid && t < tvalid;
      const int64_t idx = (row0 + t0 + t) * Dm + q.d;
      lx[i] = v ? ld_bits<T>(x, idx) : 0u;
      lr[i] = v ? ld_bits<T>(delta_raw, idx) : 0u;
      lb[i] = (t < tvalid && q.lane < N) ? ld_bits<T>(Bm, (row0 + t0 + t) * N + q.lane) : 0u;
    }
  };
  auto prep = [&](int64_t c, int buf) __attribute__((always_inline)) {
    const int tvalid = (int)(L - c * TC < TC ? L - c * TC : TC);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = q.wave + G * i;
      if (t < TC) {
        const bool v = q.dvalid && t < tvalid;
        const float delta = v ? clamp_delta(softplus_f(bits_f32<T>(lr[i]) + bias), dt_lo, dt_hi) : 0.f;
        pd[buf][t * 64 + q.lane] = make_float2(delta, delta * bits_f32<T>(lx[i]));
        if (q.lane < 16) bs[buf][t * 16 + q.lane] = bits_f32<T>(lb[i]);
      }
    }
  };
  load(q.c_begin);
  prep(q.c_begin, 0);
  if (q.c_begin + 1 < q.c_end) load(q.c_begin + 1);
  __syncthreads();
  for (int64_t c = q.c_begin; c < q.c_end; ++c) {
    const int buf = (int)((c - q.c_begin) & 1);
    if (q.dvalid) {  // state-major [b][chunk][n][d]: one coalesced row per state
#pragma unroll
      for (int j = 0; j < S; ++j)
        if (j < q.nact) hrel[((q.b * nchunks + c) * N + q.n0 + j) * Dm + q.d] = h[j];
      if (q.wave == 0) cumd[(q.b * nchunks + c) * Dm + q.d] = sd;
    }
    float2 v[TC];
    float bv[TC][S];
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      v[t] = pd[buf][t * 64 + q.lane];
#pragma unroll
      for (int j = 0; j < S; ++j) bv[t][j] = bs[buf][t * 16 + q.n0 + j];  // same address on every lane
    }
    if (c + 1 < q.c_end) {
      prep(c + 1, buf ^ 1);
      if (c + 2 < q.c_end) load(c + 2);
    }
#pragma unroll
    for (int t = 0; t < TC; ++t) {  // padded steps have Delta = 0 and B = 0
      sd += v[t].x;
#pragma unroll
      for (int j = 0; j < S; ++j) h[j] = fmaf(exp2_hw(v[t].x * A2[j]), h[j], v[t].y * bv[t][j]);
    }
    __syncthreads();
  }
  if (q.dvalid) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j < q.nact) hseg[((q.b * nseg + q.seg) * N + q.n0 + j) * Dm + q.d] = h[j];
  }
}

// ---- 2. reverse recurrence from a zero carry per segment: the carry a_t G_t leaving
// the segment's first step (same double-buffered one-barrier-per-chunk structure)
template <typename T, int S, int G, bool GATED>
__global__ void __launch_bounds__(64 * G)
seg_adj_kernel(const T* __restrict__ delta_raw, const T* __restrict__ z,
               const T* __restrict__ dy, const T* __restrict__ Cm,
               const float* __restrict__ A_log, const float* __restrict__ dt_bias,
               float* __restrict__ gseg, float* __restrict__ sdseg, int64_t L, int64_t Dm, int N, int64_t ngroups, int64_t nchunks,
               int64_t segc, int64_t nseg, float dt_lo, float dt_hi) {
  constexpr int TC = kChunk;
  constexpr int EPL = (TC + G - 1) / G;
  __shared__ float2 pa[2][TC * 64];  // (Delta, g) per (t, channel)
  __shared__ float cs[2][TC * 16];   // C per (t, state), zero beyond d_state
  Lane q = lane_setup<S>(ngroups, nseg, segc, nchunks, N);
  q.dvalid = q.d < Dm;
  const float bias = (q.dvalid && dt_bias) ? dt_bias[q.d] : 0.f;
  float A2[S], gc[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    A2[j] = (q.dvalid && j < q.nact) ? a2_from_alog(A_log[q.d * N + q.n0 + j]) : 0.f;
    gc[j] = 0.f;
  }
  float sd = 0.f;  // sum of Delta over the segment
  const int64_t row0 = q.b * L;
  // this wave's rows of a chunk (delta_raw, dy, z, C), loaded one chunk ahead of the prep
  uint32_t lr[EPL], ly[EPL], lz[EPL], lc[EPL];  // raw element bits
  auto load = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * TC;
    const int tvalid = (int)(L - t0 < TC ? L - t0 : TC);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = q.wave + G * i;
      const bool v = q.dvalid && t < tvalid;
      const int64_t idx = (row0 + t0 + t) * Dm + q.d;
      lr[i] = v ? ld_bits<T>(delta_raw, idx) : 0u;
      ly[i] = v ? ld_bits<T>(dy, idx) : 0u;
      lz[i] = (GATED && v) ? ld_bits<T>(z, idx) : 0u;
      lc[i] = (t < tvalid && q.lane < N) ? ld_bits<T>(Cm, (row0 + t0 + t) * N + q.lane) : 0u;
    }
  };
  auto prep = [&](int64_t c, int buf) __attribute__((always_inline)) {
    const int tvalid = (int)(L - c * TC < TC ? L - c * TC : TC);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = q.wave + G * i;
      if (t < TC) {
        const bool v = q.dvalid && t < tvalid;
        const float delta = v ? clamp_delta(softplus_f(bits_f32<T>(lr[i]) + bias), dt_lo, dt_hi) : 0.f;
        float g = bits_f32<T>(ly[i]);
        if (GATED) g *= silu_f(bits_f32<T>(lz[i]));
        pa[buf][t * 64 + q.lane] = make_float2(delta, g);
        if (q.lane < 16) cs[buf][t * 16 + q.lane] = bits_f32<T>(lc[i]);
      }
    }
  };
  load(q.c_end - 1);
  prep(q.c_end - 1, 0);
  if (q.c_end - 2 >= q.c_begin) load(q.c_end - 2);
  __syncthreads();
  for (int64_t c = q.c_end - 1; c >= q.c_begin; --c) {
    const int buf = (int)((q.c_end - 1 - c) & 1);
    float2 v[TC];
    float cv[TC][S];
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      v[t] = pa[buf][t * 64 + q.lane];
#pragma unroll
      for (int j = 0; j < S; ++j) cv[t][j] = cs[buf][t * 16 + q.n0 + j];  // same address on every lane
    }
    if (c - 1 >= q.c_begin) {
      prep(c - 1, buf ^ 1);
      if (c - 2 >= q.c_begin) load(c - 2);
    }
#pragma unroll
    for (int t = TC - 1; t >= 0; --t) {  // padded steps: Delta = g = 0
      sd += v[t].x;
#pragma unroll
      for (int j = 0; j < S; ++j) {
        const float Gt = fmaf(v[t].y, cv[t][j], gc[j]);  // dLoss/dh_t
        gc[j] = exp2_hw(v[t].x * A2[j]) * Gt;            // carry to h_{t-1}
      }
    }
    __syncthreads();
  }
  if (q.dvalid) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j < q.nact) gseg[((q.b * nseg + q.seg) * N + q.n0 + j) * Dm + q.d] = gc[j];
    // the segment's sum of Delta (its decay is exp(A * sum)), for the segment pass
    if (q.wave == 0) sdseg[(q.b * nseg + q.seg) * Dm + q.d] = sd;
  }
}

// ---- 3. sequential over segments per (b, d, n): state entering every segment
// (forward) and carry entering it from the right (reverse).  Segment values are
// state-major, [b][segment][n][d].
__global__ void __launch_bounds__(256)
seg_pass_kernel(const float* __restrict__ hseg, const float* __restrict__ sdseg,
                const float* __restrict__ gseg, const float* __restrict__ A_log,
                const float* __restrict__ h0, const float* __restrict__ dh_final,
                float* __restrict__ hin, float* __restrict__ gin, float* __restrict__ dh0,
                int64_t batch, int64_t Dm, int N, int64_t nseg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, n, d), d fastest
  if (i >= batch * Dm * N) return;
  const int64_t b = i / (Dm * N);
  const int n = (int)((i / Dm) % N);
  const int64_t d = i % Dm;
  const float A2 = a2_from_alog(A_log[d * N + n]);
  if (hin) {  // (skipped when the forward saved the chunk states)
    float h = h0 ? h0[(b * Dm + d) * N + n] : 0.f;
    for (int64_t s = 0; s < nseg; ++s) {
      const int64_t o = ((b * nseg + s) * N + n) * Dm + d;
      hin[o] = h;
      h = fmaf(exp2_hw(A2 * sdseg[(b * nseg + s) * Dm + d]), h, hseg[o]);
    }
  }
  // the carry beyond the last step is the gradient reaching h_final from outside; the
  // carry leaving the first segment is a_0 G_0 = dLoss/dh0
  float g = dh_final ? dh_final[(b * Dm + d) * N + n] : 0.f;
  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t o = ((b * nseg + s) * N + n) * Dm + d;
    gin[o] = g;
    g = fmaf(exp2_hw(A2 * sdseg[(b * nseg + s) * Dm + d]), g, gseg[o]);
  }
  if (dh0) dh0[(b * Dm + d) * N + n] = g;
}

// ---- 4. main backward per (b, tile, segment): chunks in reverse order
template <typename T, int S, int G, bool GATED>
__global__ void __launch_bounds__(64 * G)
bwd_main_kernel(const T* __restrict__ x, const T* __restrict__ delta_raw,
                const T* __restrict__ z, const T* __restrict__ Bm, const T* __restrict__ Cm,
                const float* __restrict__ A_log, const float* __restrict__ D_skip,
                const float* __restrict__ dt_bias, const T* __restrict__ dy,
                const float* __restrict__ hrel, const float* __restrict__ cumd,
                const float* __restrict__ hin, const float* __restrict__ gin,
                T* __restrict__ dx, T* __restrict__ ddelta_raw, T* __restrict__ dz,
                float* __restrict__ pdB, float* __restrict__ pdC, float* __restrict__ pdA,
                float* __restrict__ pdD, float* __restrict__ pdbias, int64_t L, int64_t Dm, int N,
                int64_t ngroups, int64_t nchunks, int64_t segc, int64_t nseg, float dt_lo, float dt_hi) {
  constexpr int TC = kChunk;
  constexpr int EPL = (TC + G - 1) / G;
  static_assert(2 * kSub * S == 16, "a sub-tile's dB/dC values fill one transpose-reduce");
  __shared__ float4 pd[TC * 64];                 // (Delta, Delta*x, g, -) per (t, channel)
  __shared__ float yp[TC * G * 64];              // per-wave readout partials sum_j C h
  __shared__ float2 pp[TC * G * 64];             // per-wave partials (sum G B, sum G A a h_{t-1})
  __shared__ float2 fin[G * 64];                 // per-wave dD / d_dt_bias partials
  __shared__ float2 bcs[TC * 16];                // (B, C) per (t, state), zero beyond d_state

  Lane q = lane_setup<S>(ngroups, nseg, segc, nchunks, N);
  q.dvalid = q.d < Dm;
  const int lane = q.lane, wave = q.wave;
  const int64_t b = q.b, d = q.d;
  const bool dvalid = q.dvalid;
  const int n0 = q.n0, nact = q.nact;
  const float bias = (dvalid && dt_bias) ? dt_bias[d] : 0.f;
  const float dsk = (dvalid && D_skip) ? D_skip[d] : 0.f;

  float A2[S], Av[S], Gc[S], dA[S], hi[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool v = dvalid && j < nact;
    const int64_t o = ((b * nseg + q.seg) * N + n0 + j) * Dm + d;
    Av[j] = v ? -expf(A_log[d * N + n0 + j]) : 0.f;
    A2[j] = Av[j] * kLog2e;
    Gc[j] = v ? gin[o] : 0.f;  // carry entering the segment's last step
    // state entering the segment (zero when hrel holds the forward's true chunk states)
    hi[j] = (v && hin) ? hin[o] : 0.f;
    dA[j] = 0.f;
  }
  float dD_acc = 0.f, db_acc = 0.f;
  const int64_t row0 = b * L;
  // this wave's rows of a chunk (x, delta_raw, dy, z, and B, C for lanes < d_state),
  // loaded one chunk ahead
  uint32_t lx[EPL], lr[EPL], ly[EPL], lz[EPL], lbb[EPL], lcc[EPL];  // raw element bits
  float lhr[S], lcd;  // the chunk's relative start state and Delta sum up to it
  auto load = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * TC;
    const int tvalid = (int)((L - t0) < TC ? (L - t0) : TC);
    lcd = (dvalid && cumd) ? cumd[(b * nchunks + c) * Dm + d] : 0.f;
#pragma unroll
    for (int j = 0; j < S; ++j)
      lhr[j] = (dvalid && j < nact) ? hrel[((b * nchunks + c) * N + n0 + j) * Dm + d] : 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      const bool v = dvalid && t < tvalid;
      const int64_t idx = (row0 + t0 + t) * Dm + d;
      lx[i] = v ? ld_bits<T>(x, idx) : 0u;
      lr[i] = v ? ld_bits<T>(delta_raw, idx) : 0u;
      ly[i] = v ? ld_bits<T>(dy, idx) : 0u;
      lz[i] = (GATED && v) ? ld_bits<T>(z, idx) : 0u;
      const bool ok = t < tvalid && lane < N;
      const int64_t o = (row0 + t0 + t) * N + lane;
      lbb[i] = ok ? ld_bits<T>(Bm, o) : 0u;
      lcc[i] = ok ? ld_bits<T>(Cm, o) : 0u;
    }
  };
  load(q.c_end - 1);

  for (int64_t k = q.c_end - 1; k >= q.c_begin; --k) {
    const int64_t t0 = k * TC;
    const int tvalid = (int)((L - t0) < TC ? (L - t0) : TC);
    // ---- P: per-element values (each element once, spread over all waves)
    float ex[EPL], edelta[EPL], eg[EPL], esig[EPL], egz[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      const bool v = dvalid && t < tvalid;
      const float xv = bits_f32<T>(lx[i]);
      const float r = bits_f32<T>(lr[i]) + bias;
      const float dyv = bits_f32<T>(ly[i]);
      const float sp = softplus_f(r);
      const float delta = v ? clamp_delta(sp, dt_lo, dt_hi) : 0.f;
      float g = dyv, gz = 0.f;
      if (GATED) {
        const float zv = bits_f32<T>(lz[i]);
        const float sz = sigmoid_f(zv);
        g = dyv * zv * sz;
        gz = dyv * sz * fmaf(zv, 1.f - sz, 1.f);
      }
      // d Delta / d delta_raw: the sigmoid, where the clamp lets the gradient through
      ex[i] = xv; edelta[i] = delta; eg[i] = g; esig[i] = sigmoid_f(r) * clamp_mask(sp, dt_lo, dt_hi); egz[i] = gz;
      if (t < TC) {
        pd[t * 64 + lane] = make_float4(delta, delta * xv, g, 0.f);
        if (lane < 16) bcs[t * 16 + lane] = make_float2(bits_f32<T>(lbb[i]), bits_f32<T>(lcc[i]));
      }
    }
    // start state of this chunk: relative state + decayed segment entry state
    float hs[S];
#pragma unroll
    for (int j = 0; j < S; ++j) hs[j] = fmaf(exp2_hw(A2[j] * lcd), hi[j], lhr[j]);
    if (k > q.c_begin) load(k - 1);
    __syncthreads();
    // ---- F: recompute this wave's states over the chunk, keep h_t, a_t and the
    // chunk's (Delta, Delta*x, g) in registers
    float H[TC][S], AS[TC][S];
    float4 V[TC];
    {
      float hc[S];
#pragma unroll
      for (int j = 0; j < S; ++j) hc[j] = hs[j];
#pragma unroll
      for (int t = 0; t < TC; ++t) V[t] = pd[t * 64 + lane];
#pragma unroll
      for (int t = 0; t < TC; ++t) {  // padded steps have Delta = 0 and B = C = 0
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < S; ++j) {
          const float2 bc = bcs[t * 16 + n0 + j];  // same address on every lane
          const float bj = bc.x, cj = bc.y;
          const float a = exp2_hw(V[t].x * A2[j]);
          hc[j] = fmaf(a, hc[j], V[t].y * bj);
          acc = fmaf(cj, hc[j], acc);
          AS[t][j] = a;
          H[t][j] = hc[j];
        }
        if (GATED) yp[(t * G + wave) * 64 + lane] = acc;
      }
    }
    __syncthreads();
    // ---- R1: readout s_t (fixed wave order) -> dz
    if (GATED) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int t = wave + G * i;
        if (t < tvalid && dvalid) {
          float s = dsk * ex[i];
#pragma unroll
          for (int w = 0; w < G; ++w) s += yp[(t * G + w) * 64 + lane];
          io<T>::st(dz, (row0 + t0 + t) * Dm + d, egz[i] * s);
        }
      }
    }
    // ---- V: reverse recurrence over the chunk; every kSub steps the (dB, dC) values
    // of the sub-tile are summed over the 64 channels in registers
    float red[16];
#pragma unroll
    for (int t = TC - 1; t >= 0; --t) {
      float P1 = 0.f, P2 = 0.f;
#pragma unroll
      for (int j = 0; j < S; ++j) {
        float dBp = 0.f, dCp = 0.f;
        if (j < nact) {
          const float2 bc = bcs[t * 16 + n0 + j];
          const float bj = bc.x, cj = bc.y;
          const float Gt = fmaf(V[t].z, cj, Gc[j]);      // dLoss/dh_t
          dCp = V[t].z * H[t][j];
          dBp = Gt * V[t].y;
          P1 = fmaf(Gt, bj, P1);
          const float hprev = t > 0 ? H[t - 1][j] : hs[j];
          const float w = Gt * (AS[t][j] * hprev);       // G a h_{t-1}
          dA[j] = fmaf(w, V[t].x, dA[j]);
          P2 = fmaf(w, Av[j], P2);
          Gc[j] = AS[t][j] * Gt;                          // carry to h_{t-1}
        }
        red[2 * ((t % kSub) * S + j)] = dBp;
        red[2 * ((t % kSub) * S + j) + 1] = dCp;
      }
      pp[(t * G + wave) * 64 + lane] = make_float2(P1, P2);
      if (t % kSub == 0) {
        // lane i holds the channel sum of value (i >> 2) & 15 = 2 * (step * S + state) + (0: dB, 1: dC)
        const float sum = transpose_reduce16(red, lane);
        const int o16 = (lane >> 2) & 15;
        const int pidx = o16 >> 1, j = pidx % S;
        const int ts = t + pidx / S;  // absolute step inside the chunk
        if ((lane & 3) == 0 && j < nact && ts < tvalid) {
          const int64_t o = ((b * ngroups + q.grp) * L + t0 + ts) * N + n0 + j;
          ((o16 & 1) ? pdC : pdB)[o] = sum;
        }
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
          const float2 qv = pp[(t * G + w) * 64 + lane];
          P1 += qv.x;
          P2 += qv.y;
        }
        const int64_t idx = (row0 + t0 + t) * Dm + d;
        io<T>::st(dx, idx, fmaf(eg[i], dsk, edelta[i] * P1));
        const float dr = fmaf(ex[i], P1, P2) * esig[i];
        io<T>::st(ddelta_raw, idx, dr);
        dD_acc = fmaf(eg[i], ex[i], dD_acc);
        db_acc += dr;
      }
    }
    __syncthreads();
  }
  // ---- per-(b, segment, d) partials: dA raw sums, and dD / d_dt_bias joined over
  // waves in order
  const int64_t po = (b * nseg + q.seg) * Dm + d;
  if (dvalid) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j < nact) pdA[((b * nseg + q.seg) * N + n0 + j) * Dm + d] = dA[j];
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
    pdD[po] = sD;
    pdbias[po] = sb;
  }
}

// ---- 5a. dB, dC: sum of the channel-tile partials in ascending tile order
__global__ void __launch_bounds__(256)
reduce_bc_kernel(const float* __restrict__ pdB, const float* __restrict__ pdC, float* __restrict__ dB,
                 float* __restrict__ dC, int64_t batch, int64_t L, int N, int64_t ngroups) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, t, n)
  const int64_t per_b = L * N;
  if (i >= batch * per_b) return;
  const int64_t b = i / per_b, tn = i % per_b;
  const float* pb = pdB + b * ngroups * per_b + tn;
  const float* pc = pdC + b * ngroups * per_b + tn;
  float sB = 0.f, sC = 0.f;
  int64_t g = 0;
  // eight tiles' loads in flight at a time, added in ascending tile order
  for (; g + 8 <= ngroups; g += 8) {
    float vb[8], vc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      vb[k] = pb[(g + k) * per_b];
      vc[k] = pc[(g + k) * per_b];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sB += vb[k];
      sC += vc[k];
    }
  }
  for (; g < ngroups; ++g) {
    sB += pb[g * per_b];
    sC += pc[g * per_b];
  }
  dB[i] = sB;
  dC[i] = sC;
}

// ---- 5b. dA_log, dD, d_dt_bias: sums over (batch, segment) in lexical order
__global__ void __launch_bounds__(256)
reduce_params_kernel(const float* __restrict__ pdA, const float* __restrict__ pdD,
                     const float* __restrict__ pdbias, const float* __restrict__ A_log,
                     float* __restrict__ dA_log, float* __restrict__ dD, float* __restrict__ d_dt_bias,
                     int64_t nparts, int64_t Dm, int N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (n, d), d fastest
  if (i < Dm * N && dA_log) {
    const int64_t n = i / Dm, d = i % Dm;
    float s = 0.f;
#pragma unroll 8
    for (int64_t p = 0; p < nparts; ++p) s += pdA[p * Dm * N + i];  // partials are [part][n][d]
    dA_log[d * N + n] = s * -expf(A_log[d * N + n]);                // dA/dA_log = A
  }
  if (i < Dm) {
    float sD = 0.f, sb = 0.f;
#pragma unroll 8
    for (int64_t p = 0; p < nparts; ++p) {
      sD += pdD[p * Dm + i];
      sb += pdbias[p * Dm + i];
    }
    if (dD) dD[i] = sD;
    if (d_dt_bias) d_dt_bias[i] = sb;
  }
}

template <typename T, int G>
hipError_t launch_segments(const BwdArgs& a, const BwdLayout& l, char* ws, hipStream_t stream) {
  const T *x = (const T*)a.x, *dr = (const T*)a.delta_raw, *z = (const T*)a.z, *dy = (const T*)a.dy;
  const T *Bm = (const T*)a.B, *Cm = (const T*)a.C;
  T *dx = (T*)a.dx, *ddr = (T*)a.ddelta_raw, *dz = (T*)a.dz;
  constexpr int S = kS;
  const unsigned blocks = (unsigned)(a.batch * l.nseg * l.ngroups);
  // With the forward's saved chunk states (the true state entering every chunk, in
  // hrel's layout) the chunk-relative forward pass and the state half of the segment
  // pass are skipped: bwd_main reads the saved states as start states, with a zero
  // Delta sum and a zero segment entry state.
  const bool saved = a.chunk_states != nullptr;
  float* hrel = saved ? const_cast<float*>(a.chunk_states) : (float*)(ws + l.off_hrel);
  float* cumd = saved ? nullptr : (float*)(ws + l.off_cumd);
  float* hseg = saved ? nullptr : (float*)(ws + l.off_hseg);
  float* sdseg = (float*)(ws + l.off_sdseg);
  float* gseg = (float*)(ws + l.off_gseg);
  float* hin = saved ? nullptr : (float*)(ws + l.off_hin);
  float* gin = (float*)(ws + l.off_gin);
  hipError_t e;
  if (!saved) {
    hipLaunchKernelGGL((chunk_rel_kernel<T, S, G>), dim3(blocks), dim3(64 * G), 0, stream, x, dr, Bm,
                       a.A_log, a.dt_bias, hrel, cumd, hseg, a.seqlen, a.dim, a.dstate, l.ngroups,
                       l.nchunks, l.segc, l.nseg, a.dt_lo, a.dt_hi);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.z)
    hipLaunchKernelGGL((seg_adj_kernel<T, S, G, true>), dim3(blocks), dim3(64 * G), 0, stream, dr, z,
                       dy, Cm, a.A_log, a.dt_bias, gseg, sdseg, a.seqlen, a.dim, a.dstate, l.ngroups,
                       l.nchunks, l.segc, l.nseg, a.dt_lo, a.dt_hi);
  else
    hipLaunchKernelGGL((seg_adj_kernel<T, S, G, false>), dim3(blocks), dim3(64 * G), 0, stream, dr, z,
                       dy, Cm, a.A_log, a.dt_bias, gseg, sdseg, a.seqlen, a.dim, a.dstate, l.ngroups,
                       l.nchunks, l.segc, l.nseg, a.dt_lo, a.dt_hi);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    const int64_t n = a.batch * a.dim * a.dstate;
    hipLaunchKernelGGL(seg_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, hseg, sdseg,
                       gseg, a.A_log, a.h0, a.dh_final, hin, gin, a.dh0, a.batch, a.dim, a.dstate, l.nseg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  float* pdB = (float*)(ws + l.off_dbc);
  float* pdC = pdB + (size_t)a.batch * l.ngroups * a.seqlen * a.dstate;
  float* pdA = (float*)(ws + l.off_dparam);
  float* pdD = pdA + (size_t)a.batch * l.nseg * a.dim * a.dstate;
  float* pdb = pdD + (size_t)a.batch * l.nseg * a.dim;
  if (a.z)
    hipLaunchKernelGGL((bwd_main_kernel<T, S, G, true>), dim3(blocks), dim3(64 * G), 0, stream, x,
                       dr, z, Bm, Cm, a.A_log, a.D_skip, a.dt_bias, dy, hrel, cumd, hin, gin,
                       dx, ddr, dz, pdB, pdC, pdA, pdD, pdb, a.seqlen, a.dim, a.dstate,
                       l.ngroups, l.nchunks, l.segc, l.nseg, a.dt_lo, a.dt_hi);
  else
    hipLaunchKernelGGL((bwd_main_kernel<T, S, G, false>), dim3(blocks), dim3(64 * G), 0, stream, x,
                       dr, z, Bm, Cm, a.A_log, a.D_skip, a.dt_bias, dy, hrel, cumd, hin, gin,
                       dx, ddr, dz, pdB, pdC, pdA, pdD, pdb, a.seqlen, a.dim, a.dstate,
                       l.ngroups, l.nchunks, l.segc, l.nseg, a.dt_lo, a.dt_hi);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, void* workspace, hipStream_t stream) {
  const BwdLayout l = bwd_layout(a.batch, a.seqlen, a.dim, a.dstate);
  char* ws = (char*)workspace;
  hipError_t e;
  if (l.fused) {
    const float* cs = a.chunk_states;
    if (!cs) {  // the forward did not save its chunk states: a states-only forward writes them
      FwdArgs f;
      f.x = a.x; f.delta_raw = a.delta_raw; f.z = nullptr; f.B = a.B; f.C = a.C; f.A_log = a.A_log;
      f.D_skip = nullptr; f.dt_bias = a.dt_bias; f.h0 = a.h0; f.y = nullptr; f.h_final = nullptr;
      f.batch = a.batch; f.seqlen = a.seqlen; f.dim = a.dim; f.dstate = a.dstate; f.bf16 = a.bf16;
      f.dt_lo = a.dt_lo; f.dt_hi = a.dt_hi; f.chunk_states = (float*)(ws + l.off_cs);
      if ((e = launch_fwd_states(f, stream)) != hipSuccess) return e;
      cs = f.chunk_states;
    }
    float* pdB = (float*)(ws + l.off_dbc);
    float* pdC = pdB + (size_t)a.batch * l.ngroups * a.seqlen * a.dstate;
    float* pdA = (float*)(ws + l.off_dparam);
    float* pdD = pdA + (size_t)a.batch * a.dim * a.dstate;
    float* pdb = pdD + (size_t)a.batch * a.dim;
    if ((e = launch_bwd_fused(a, cs, pdB, pdC, pdA, pdD, pdb, stream)) != hipSuccess) return e;
    const int64_t n = a.batch * a.seqlen * a.dstate;
    hipLaunchKernelGGL(reduce_bc_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, pdB, pdC,
                       a.dB, a.dC, a.batch, a.seqlen, a.dstate, l.ngroups);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t np = a.dim * a.dstate > a.dim ? a.dim * a.dstate : a.dim;
    hipLaunchKernelGGL(reduce_params_kernel, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, stream, pdA, pdD,
                       pdb, a.A_log, a.dA_log, a.dD, a.d_dt_bias, a.batch, a.dim, a.dstate);
    return hipGetLastError();
  }
  switch (waves_for(a.dstate)) {
    case 1: e = a.bf16 ? launch_segments<bf16_t, 1>(a, l, ws, stream) : launch_segments<float, 1>(a, l, ws, stream); break;
    case 2: e = a.bf16 ? launch_segments<bf16_t, 2>(a, l, ws, stream) : launch_segments<float, 2>(a, l, ws, stream); break;
    case 4: e = a.bf16 ? launch_segments<bf16_t, 4>(a, l, ws, stream) : launch_segments<float, 4>(a, l, ws, stream); break;
    default: e = a.bf16 ? launch_segments<bf16_t, 8>(a, l, ws, stream) : launch_segments<float, 8>(a, l, ws, stream); break;
  }
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
    float* pdD = pdA + (size_t)a.batch * l.nseg * a.dim * a.dstate;
    float* pdb = pdD + (size_t)a.batch * l.nseg * a.dim;
    const int64_t n = a.dim * a.dstate > a.dim ? a.dim * a.dstate : a.dim;
    hipLaunchKernelGGL(reduce_params_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, pdA, pdD,
                       pdb, a.A_log, a.dA_log, a.dD, a.d_dt_bias, a.batch * l.nseg, a.dim, a.dstate);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ssm
