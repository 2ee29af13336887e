// ssm_fwd.hip -- forward selective scan for gfx950.
//
// Computes, for every (batch b, channel d), the recurrence of the POPCORNBENCH
// transcript's selective_scan_kernel (state update first, readout from the updated
// state, skip term) with the discretisation and gate of mamba-rs kernels.rs
// (softplus_fwd / exp_negate / split_gate_silu, gating_backward: y = ssm_out * gate):
//   Delta = softplus(delta_raw + dt_bias), a = exp(Delta A) = exp2(Delta A2)
//   h_n  <- a h_n + (Delta x) B_n ;  y = (sum_n C_n h_n + D x) * silu(z)
//
// Work decomposition (designed for 64-lane wavefronts, not taken from the pages):
//   * one workgroup = one batch element b and a tile of 64 consecutive channels;
//     lane = channel, so every global load and store of x/delta_raw/z/y is one
//     contiguous 256 B (fp32) or 128 B (bf16) row segment per wavefront;
//   * the G wavefronts of the workgroup split the state axis: wave w owns states
//     [w*S, w*S + S) of all 64 channels and keeps them in VGPRs for the whole
//     sequence.  All 64 lanes of a wave need the same B[b,t,n] and C[b,t,n], so
//     those are wave-uniform scalar loads (SGPR operands, no VALU or LDS cost);
//   * per-(t,d) work (softplus, Delta*x, D*x, silu(z)) is done once per element
//     in a "prep" phase spread over all waves and shared through LDS, and the
//     readout sum over states is a per-wave partial in LDS that a "readout"
//     phase adds in fixed wave order -- so the result is deterministic.
// Time is walked in tiles of TT steps: prep(k) | barrier | scan(k) | barrier |
// readout(k), with the global loads of tile k+1 issued right after prep(k) so
// their latency hides behind scan(k).
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

template <typename T, int S, int G, int TT, bool GATED>
__global__ void __launch_bounds__(64 * G)
fwd_scan_kernel(const T* __restrict__ x, const T* __restrict__ delta_raw, const T* __restrict__ z,
                const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ A_log,
                const float* __restrict__ D_skip, const float* __restrict__ dt_bias,
                const float* __restrict__ h0, T* __restrict__ y, float* __restrict__ h_final,
                int64_t L, int64_t Dm, int N, int64_t ngroups) {
  constexpr int EPL = (TT + G - 1) / G;  // prep/readout elements per lane per tile
  __shared__ float2 dd[TT * 64];         // (Delta, Delta*x) per (t, channel)
  __shared__ float yp[TT * G * 64];      // per-wave partial readout per (t, wave, channel)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.x / ngroups;
  const int64_t d = (blockIdx.x % ngroups) * 64 + lane;
  const bool dvalid = d < Dm;
  const float bias = (dvalid && dt_bias) ? dt_bias[d] : 0.f;
  const float dsk = (dvalid && D_skip) ? D_skip[d] : 0.f;

  const int n0 = wave * S;
  const int nact = N - n0 < 0 ? 0 : (N - n0 > S ? S : N - n0);  // wave-uniform
  float A2[S], h[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool v = dvalid && j < nact;
    A2[j] = v ? a2_from_alog(A_log[d * N + n0 + j]) : 0.f;
    h[j] = (v && h0) ? h0[(b * Dm + d) * N + n0 + j] : 0.f;
  }

  const int64_t row0 = b * L;  // row of (b, t) is row0 + t
  float px[EPL], pr[EPL], pz[EPL];
  auto load_tile = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      const bool v = dvalid && t < TT && t0 + t < L;
      const int64_t idx = (row0 + t0 + t) * Dm + d;
      px[i] = v ? io<T>::ld(x, idx) : 0.f;
      pr[i] = v ? io<T>::ld(delta_raw, idx) : 0.f;
      pz[i] = (GATED && v) ? io<T>::ld(z, idx) : 0.f;
    }
  };

  const int64_t ntiles = (L + TT - 1) / TT;
  load_tile(0);
  for (int64_t k = 0; k < ntiles; ++k) {
    const int64_t t0 = k * TT;
    const int tvalid = (int)((L - t0) < TT ? (L - t0) : TT);
    // ---- prep: Delta, Delta*x into LDS; skip term and gate kept in registers
    float skip[EPL], gate[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      if (t < TT) {
        const bool v = dvalid && t < tvalid;
        const float delta = softplus_f(pr[i] + bias);
        dd[t * 64 + lane] = v ? make_float2(delta, delta * px[i]) : make_float2(0.f, 0.f);
        skip[i] = dsk * px[i];
        gate[i] = GATED ? silu_f(pz[i]) : 1.f;
      }
    }
    if (k + 1 < ntiles) load_tile(t0 + TT);
    __syncthreads();
    // ---- scan: this wave's states over the tile
    {
      const T* __restrict__ Bt = Bm + (row0 + t0) * N + n0;
      const T* __restrict__ Ct = Cm + (row0 + t0) * N + n0;
      float* __restrict__ ypw = yp + wave * 64 + lane;
      if (nact == S) {
        for (int t = 0; t < tvalid; ++t) {
          const float2 v = dd[t * 64 + lane];
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < S; ++j) {
            const float a = exp2_hw(v.x * A2[j]);
            h[j] = fmaf(a, h[j], v.y * io<T>::ld(Bt, t * N + j));
            acc = fmaf(io<T>::ld(Ct, t * N + j), h[j], acc);
          }
          ypw[t * G * 64] = acc;
        }
      } else {
        for (int t = 0; t < tvalid; ++t) {
          const float2 v = dd[t * 64 + lane];
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < S; ++j) {
            if (j < nact) {
              const float a = exp2_hw(v.x * A2[j]);
              h[j] = fmaf(a, h[j], v.y * io<T>::ld(Bt, t * N + j));
              acc = fmaf(io<T>::ld(Ct, t * N + j), h[j], acc);
            }
          }
          ypw[t * G * 64] = acc;
        }
      }
    }
    __syncthreads();
    // ---- readout: add the wave partials in fixed order, skip term, gate, store
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      if (t < tvalid && dvalid) {
        float s = skip[i];
#pragma unroll
        for (int w = 0; w < G; ++w) s += yp[(t * G + w) * 64 + lane];
        io<T>::st(y, (row0 + t0 + t) * Dm + d, s * gate[i]);
      }
    }
  }
  if (h_final && dvalid) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j < nact) h_final[(b * Dm + d) * N + n0 + j] = h[j];
  }
}

template <typename T, int S, int G, bool GATED>
hipError_t launch_cfg(const FwdArgs& a, hipStream_t stream) {
  constexpr int TT = 16;
  const int64_t ngroups = (a.dim + 63) / 64;
  const int64_t nblocks = ngroups * a.batch;
  hipLaunchKernelGGL((fwd_scan_kernel<T, S, G, TT, GATED>), dim3((unsigned)nblocks), dim3(64 * G), 0,
                     stream, (const T*)a.x, (const T*)a.delta_raw, (const T*)a.z, (const T*)a.B,
                     (const T*)a.C, a.A_log, a.D_skip, a.dt_bias, a.h0, (T*)a.y, a.h_final, a.seqlen,
                     a.dim, a.dstate, ngroups);
  return hipGetLastError();
}

// States per wave S: fewer states per wave means more wavefronts (more parallelism)
// but more LDS traffic per state update.  Default: two states per wave.
int pick_states_per_wave(const FwdArgs& a, int ns) {
  if (const char* e = getenv("SSM_FWD_STATES_PER_WAVE")) {
    const int v = atoi(e);
    if (v == 1 || v == 2 || v == 4 || v == ns) return v;
  }
  return ns == 4 ? 1 : 2;
}

template <typename T, bool GATED>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int ns = a.dstate <= 4 ? 4 : (a.dstate <= 8 ? 8 : 16);
  const int s = pick_states_per_wave(a, ns);
  if (ns == 16) {
    switch (s) {
      case 1: return launch_cfg<T, 1, 16, GATED>(a, stream);
      case 4: return launch_cfg<T, 4, 4, GATED>(a, stream);
      case 16: return launch_cfg<T, 16, 1, GATED>(a, stream);
      default: return launch_cfg<T, 2, 8, GATED>(a, stream);
    }
  }
  if (ns == 8) {
    switch (s) {
      case 1: return launch_cfg<T, 1, 8, GATED>(a, stream);
      case 8: return launch_cfg<T, 8, 1, GATED>(a, stream);
      default: return launch_cfg<T, 2, 4, GATED>(a, stream);
    }
  }
  switch (s) {
    case 4: return launch_cfg<T, 4, 1, GATED>(a, stream);
    default: return launch_cfg<T, 1, 4, GATED>(a, stream);
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.bf16) return a.z ? launch_t<bf16_t, true>(a, stream) : launch_t<bf16_t, false>(a, stream);
  return a.z ? launch_t<float, true>(a, stream) : launch_t<float, false>(a, stream);
}

}  // namespace ssm
