// ssm_step.hip -- single-step decode update (mamba-rs kernels.rs, MambaKernels field
// ssm_step_fwd: the SSM forward for one time step, used at inference), state updated
// in place.
//
// The step is bound by HBM traffic of the state (read + write of batch*d_inner*d_state
// fp32), so the layout is chosen for that stream: QL lanes share one (b, d) pair and
// each lane owns 4 consecutive states, so consecutive lanes touch consecutive 16 B of
// the state and every wavefront reads and writes one contiguous block.  The readout
// sum over states is a fixed-order butterfly over the QL lanes of a pair.
//
// CONV (the decode step of a Mamba block): the token first goes through the depthwise
// causal conv1d step, computed as the conv1d step kernel computes it: the K-tap window
// is the conv state's K - 1 entries followed by the token, p = bias + sum over k in
// ascending order of w[d][k] window[k] (fused multiply-adds), then SiLU if asked.  p
// is rounded to the I/O type, as a separate conv step would store it and the scan
// step read it back, and takes the place of x, so results are bit-identical to the two
// calls.  Every lane of a (b, d) pair loads the window and the weights with the scan's
// operands (no value is used before every load of the step has gone out) and forms p;
// lane 0 of the pair shifts the conv state from its registers and stores p when asked.
// The width K is a template parameter (0: no convolution), so that the taps' loads and
// stores merge into wide accesses.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

// a value as the I/O type stores it, read back
template <typename T> __device__ __forceinline__ float as_io(float v);
template <> __device__ __forceinline__ float as_io<float>(float v) { return v; }
template <> __device__ __forceinline__ float as_io<bf16_t>(float v) { return bf16_to_f32(f32_to_bf16(v)); }

template <typename T, int QL, bool VEC, bool GATED, int K>
__global__ void __launch_bounds__(256)
step_kernel(float* __restrict__ state, const T* __restrict__ x, const T* __restrict__ delta_raw,
            const T* __restrict__ z, const T* __restrict__ Bm, const T* __restrict__ Cm,
            const float* __restrict__ A_log, const float* __restrict__ D_skip,
            const float* __restrict__ dt_bias, T* __restrict__ y, int64_t batch, int64_t Dm, int N,
            float dt_lo, float dt_hi, T* __restrict__ cstate, const float* __restrict__ cw,
            const float* __restrict__ cb, T* __restrict__ u, bool silu) {
  constexpr bool CONV = K > 0;
  constexpr int KS = K > 1 ? K - 1 : 1, KW = K > 0 ? K : 1;  // array sizes
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = gid / QL;  // (b, d) flattened: b * Dm + d
  const int q = (int)(gid % QL);
  const bool valid = pair < batch * Dm;
  const int64_t b = valid ? pair / Dm : 0;
  const int64_t d = valid ? pair % Dm : 0;
  const int n0 = q * 4;
  int nv = N - n0;
  nv = valid ? (nv < 0 ? 0 : (nv > 4 ? 4 : nv)) : 0;

  float xv = 0.f, rv = 0.f, zv = 0.f, bias = 0.f, dsk = 0.f;
  // CONV: the conv state's K - 1 entries, the token, the weights and the bias (no value
  // is used before every load of the step has gone out)
  float sv[KS], wk[KW], xt = 0.f, cbias = 0.f;
  T* const cs = CONV ? cstate + pair * (K - 1) : nullptr;
  if (valid) {
    if (CONV) {
      xt = io<T>::ld(x, pair);
#pragma unroll
      for (int k = 0; k < K - 1; ++k) sv[k] = io<T>::ld(cs, k);
#pragma unroll
      for (int k = 0; k < K; ++k) wk[k] = cw[d * K + k];
      if (cb) cbias = cb[d];
    } else {
      xv = io<T>::ld(x, pair);
    }
    rv = io<T>::ld(delta_raw, pair);
    if (GATED) zv = io<T>::ld(z, pair);
    if (dt_bias) bias = dt_bias[d];
    if (D_skip) dsk = D_skip[d];
  }
  float h[4] = {0.f, 0.f, 0.f, 0.f}, al[4] = {0.f, 0.f, 0.f, 0.f};
  float bv[4] = {0.f, 0.f, 0.f, 0.f}, cv[4] = {0.f, 0.f, 0.f, 0.f};
  float* __restrict__ st = state + pair * N + n0;
  if (VEC) {
    if (nv == 4) {
      const float4 s4 = *reinterpret_cast<const float4*>(st);
      const float4 a4 = *reinterpret_cast<const float4*>(A_log + d * N + n0);
      h[0] = s4.x; h[1] = s4.y; h[2] = s4.z; h[3] = s4.w;
      al[0] = a4.x; al[1] = a4.y; al[2] = a4.z; al[3] = a4.w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bv[j] = io<T>::ld(Bm, b * N + n0 + j);
        cv[j] = io<T>::ld(Cm, b * N + n0 + j);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < nv) {
        h[j] = st[j];
        al[j] = A_log[d * N + n0 + j];
        bv[j] = io<T>::ld(Bm, b * N + n0 + j);
        cv[j] = io<T>::ld(Cm, b * N + n0 + j);
      }
    }
  }
  // the window: the conv state's entries, then the token
  auto win = [&](int k) __attribute__((always_inline)) { return k < K - 1 ? sv[k] : xt; };
  float p = 0.f;
  if (CONV && valid) {
    p = cbias;
#pragma unroll
    for (int k = 0; k < K; ++k) p = fmaf(wk[k], win(k), p);
    if (silu) p = silu_f(p);
    xv = as_io<T>(p);
  }
  const float delta = clamp_delta(softplus_f(rv + bias), dt_lo, dt_hi);
  const float dx = delta * xv;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < nv) {
      const float a = exp2_hw(delta * a2_from_alog(al[j]));
      h[j] = fmaf(a, h[j], dx * bv[j]);
      acc = fmaf(cv[j], h[j], acc);
    }
  }
  if (VEC) {
    if (nv == 4) *reinterpret_cast<float4*>(st) = make_float4(h[0], h[1], h[2], h[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nv) st[j] = h[j];
  }
  // fixed-order butterfly over the QL lanes of this pair (all lanes take part)
  if (QL >= 2) acc += __shfl_xor(acc, 1, QL);
  if (QL >= 4) acc += __shfl_xor(acc, 2, QL);
  if (CONV && valid && q == 0) {  // the conv state shifted by one token, from registers
#pragma unroll
    for (int k = 0; k < K - 1; ++k) io<T>::st(cs, k, win(k + 1));
    if (u) io<T>::st(u, pair, p);
  }
  if (valid && q == 0) {
    const float s = acc + dsk * xv;
    io<T>::st(y, pair, GATED ? s * silu_f(zv) : s);
  }
}

template <typename T, int QL, bool GATED, int K>
hipError_t launch_qlk(const StepArgs& a, bool vec, hipStream_t stream) {
  const int64_t threads = a.batch * a.dim * QL;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  auto kern = vec ? step_kernel<T, QL, true, GATED, K> : step_kernel<T, QL, false, GATED, K>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, stream, a.state, (const T*)a.x, (const T*)a.delta_raw,
                     (const T*)a.z, (const T*)a.B, (const T*)a.C, a.A_log, a.D_skip, a.dt_bias, (T*)a.y, a.batch,
                     a.dim, a.dstate, a.dt_lo, a.dt_hi, (T*)a.conv_state, a.conv_w, a.conv_b, (T*)a.u, a.silu);
  return hipGetLastError();
}
template <typename T, int QL, bool GATED>
hipError_t launch_ql(const StepArgs& a, bool vec, hipStream_t stream) {
  switch (a.width) {
    case 0: return launch_qlk<T, QL, GATED, 0>(a, vec, stream);
    case 1: return launch_qlk<T, QL, GATED, 1>(a, vec, stream);
    case 2: return launch_qlk<T, QL, GATED, 2>(a, vec, stream);
    case 3: return launch_qlk<T, QL, GATED, 3>(a, vec, stream);
    case 4: return launch_qlk<T, QL, GATED, 4>(a, vec, stream);
    case 5: return launch_qlk<T, QL, GATED, 5>(a, vec, stream);
    case 6: return launch_qlk<T, QL, GATED, 6>(a, vec, stream);
    case 7: return launch_qlk<T, QL, GATED, 7>(a, vec, stream);
    default: return launch_qlk<T, QL, GATED, 8>(a, vec, stream);
  }
}

template <typename T, bool GATED>
hipError_t launch_t(const StepArgs& a, hipStream_t stream) {
  // float4 state and A_log accesses need d_state % 4 == 0 and 16 B aligned bases
  const bool vec = (a.dstate % 4 == 0) && ((uintptr_t)a.state % 16 == 0) && ((uintptr_t)a.A_log % 16 == 0);
  if (a.dstate <= 4) return launch_ql<T, 1, GATED>(a, vec, stream);
  if (a.dstate <= 8) return launch_ql<T, 2, GATED>(a, vec, stream);
  return launch_ql<T, 4, GATED>(a, vec, stream);
}

}  // namespace

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  if (a.bf16) return a.z ? launch_t<bf16_t, true>(a, stream) : launch_t<bf16_t, false>(a, stream);
  return a.z ? launch_t<float, true>(a, stream) : launch_t<float, false>(a, stream);
}

}  // namespace ssm
