// ssm_conv1d.hip -- depthwise causal conv1d (+ optional SiLU) for gfx950: the
// step before the selective scan in a Mamba block (mamba-rs kernels.rs, MambaKernels
// conv1d fields: conv1d_step_fwd, the one-step decode conv with SiLU;
// conv1d_burnin_fwd, the multi-step forward; conv1d_step_bwd / conv1d_burnin_bwd).
//   p[b,t,d] = sum_{k<K} w[d,k] x[b,t-(K-1)+k,d] + bias[d]   (no history before t = 0)
//   out      = silu(p) or p
// The weight and bias gradients are fixed-order sums of per-(batch, time tile)
// partials, added in lexical order (deterministic_backward.py, ordered_conv: per-batch
// partials summed in batch order, no atomics).
//
// All three kernels are HBM streams: lane = channel, so every load and store of a
// [B, L, D] row is one contiguous 256 B (fp32) / 128 B (bf16) segment per wavefront,
// and each lane walks a tile of TL time steps keeping the K-tap window in registers
// (the halo of K-1 rows per tile is the only re-read).  All loads of a tile are
// issued before any arithmetic.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kFwdTile = 32;  // time steps per lane in the forward
constexpr int kBwdTile = 16;  // time steps per lane in the backward
constexpr int kWaves = 4;     // wavefronts per workgroup, one time tile each

template <typename T, int K, bool SILU>
__global__ void __launch_bounds__(64 * kWaves)
conv_fwd_kernel(const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
                T* __restrict__ out, int64_t L, int64_t Dm, int64_t ngroups, int64_t ntg) {
  constexpr int TL = kFwdTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // block -> (b, time group, channel group), channel groups fastest
  const int64_t grp = blockIdx.x % ngroups;
  const int64_t r = blockIdx.x / ngroups;
  const int64_t tg = r % ntg, b = r / ntg;
  const int64_t d = grp * 64 + lane;
  const int64_t t0 = (tg * kWaves + wave) * TL;
  if (d >= Dm || t0 >= L) return;  // no barriers in this kernel
  float wk[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wk[k] = w[d * K + k];
  const float bs = bias ? bias[d] : 0.f;
  // x[t0-K+1 .. t0+TL-1], zero before t = 0 and past the end
  float xr[TL + K - 1];
#pragma unroll
  for (int i = 0; i < TL + K - 1; ++i) {
    const int64_t t = t0 - (K - 1) + i;
    xr[i] = (t >= 0 && t < L) ? io<T>::ld(x, (b * L + t) * Dm + d) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    float p = bs;
#pragma unroll
    for (int k = 0; k < K; ++k) p = fmaf(wk[k], xr[i + k], p);
    if (t0 + i < L) io<T>::st(out, (b * L + t0 + i) * Dm + d, SILU ? silu_f(p) : p);
  }
}

template <typename T, int K, bool SILU>
__global__ void __launch_bounds__(256)
conv_step_kernel(T* __restrict__ state, const T* __restrict__ x, const float* __restrict__ w,
                 const float* __restrict__ bias, T* __restrict__ out, int64_t batch, int64_t Dm) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, d)
  if (i >= batch * Dm) return;
  const int64_t d = i % Dm;
  float win[K];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) win[k] = io<T>::ld(state, i * (K - 1) + k);
  win[K - 1] = io<T>::ld(x, i);
  float p = bias ? bias[d] : 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) p = fmaf(w[d * K + k], win[k], p);
  io<T>::st(out, i, SILU ? silu_f(p) : p);
#pragma unroll
  for (int k = 0; k < K - 1; ++k) io<T>::st(state, i * (K - 1) + k, win[k + 1]);
}

// backward of one (b, time tile, channel): dx for the tile, and the tile's partial
// dw[k] = sum_t dp[t] x[t-K+1+k] and dbias = sum_t dp[t], stored [b][tile][k][d]
template <int K, bool SILU>
__global__ void __launch_bounds__(64 * kWaves)
conv_bwd_kernel(const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
                const float* __restrict__ dout, float* __restrict__ dx, float* __restrict__ pdw,
                float* __restrict__ pdb, int64_t L, int64_t Dm, int64_t ngroups, int64_t ntg, int64_t ntiles) {
  constexpr int TL = kBwdTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t grp = blockIdx.x % ngroups;
  const int64_t r = blockIdx.x / ngroups;
  const int64_t tg = r % ntg, b = r / ntg;
  const int64_t d = grp * 64 + lane;
  const int64_t tile = tg * kWaves + wave;
  const int64_t t0 = tile * TL;
  if (d >= Dm || t0 >= L) return;  // no barriers in this kernel
  float wk[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wk[k] = w[d * K + k];
  const float bs = bias ? bias[d] : 0.f;
  // x[t0-K+1 .. t0+TL+K-2] and dout[t0 .. t0+TL+K-2], zero outside the sequence
  constexpr int NX = TL + 2 * (K - 1), NG = TL + K - 1;
  float xr[NX], gr[NG];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int64_t t = t0 - (K - 1) + i;
    xr[i] = (t >= 0 && t < L) ? x[(b * L + t) * Dm + d] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int64_t t = t0 + i;
    gr[i] = t < L ? dout[(b * L + t) * Dm + d] : 0.f;
  }
  // dp[t0 + i] for i < TL + K - 1 (dp = 0 past the end since dout = 0 there)
  float dp[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    if (SILU) {
      float p = bs;
#pragma unroll
      for (int k = 0; k < K; ++k) p = fmaf(wk[k], xr[i + k], p);
      const float sg = sigmoid_f(p);
      dp[i] = gr[i] * sg * fmaf(p, 1.f - sg, 1.f);
    } else {
      dp[i] = gr[i];
    }
  }
  float sw[K], sb = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) sw[k] = 0.f;
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    float g = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) g = fmaf(wk[k], dp[i + K - 1 - k], g);
    if (t0 + i < L) dx[(b * L + t0 + i) * Dm + d] = g;
    // the tile's own steps only (dp of the halo belongs to the next tile)
#pragma unroll
    for (int k = 0; k < K; ++k) sw[k] = fmaf(dp[i], xr[i + k], sw[k]);
    sb += dp[i];
  }
  const int64_t o = (b * ntiles + tile) * K;
#pragma unroll
  for (int k = 0; k < K; ++k) pdw[(o + k) * Dm + d] = sw[k];
  pdb[(b * ntiles + tile) * Dm + d] = sb;
}

// dw[d,k] and dbias[d]: sums of the partials over (b, tile) in lexical order
template <int K>
__global__ void __launch_bounds__(256)
conv_reduce_kernel(const float* __restrict__ pdw, const float* __restrict__ pdb, float* __restrict__ dw,
                   float* __restrict__ dbias, int64_t nparts, int64_t Dm) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (k, d), d fastest
  if (i < K * Dm && dw) {
    const int64_t k = i / Dm, d = i % Dm;
    float s = 0.f;
#pragma unroll 8
    for (int64_t p = 0; p < nparts; ++p) s += pdw[p * K * Dm + i];
    dw[d * K + k] = s;
  }
  if (i < Dm && dbias) {
    float s = 0.f;
#pragma unroll 8
    for (int64_t p = 0; p < nparts; ++p) s += pdb[p * Dm + i];
    dbias[i] = s;
  }
}

template <typename T, int K>
hipError_t fwd_k(const ConvArgs& a, hipStream_t stream) {
  const int64_t ngroups = (a.dim + 63) / 64;
  const int64_t ntg = (a.seqlen + kFwdTile * kWaves - 1) / (kFwdTile * kWaves);
  const dim3 grid((unsigned)(ngroups * ntg * a.batch));
  if (a.silu)
    hipLaunchKernelGGL((conv_fwd_kernel<T, K, true>), grid, dim3(64 * kWaves), 0, stream, (const T*)a.x, a.w,
                       a.bias, (T*)a.out, a.seqlen, a.dim, ngroups, ntg);
  else
    hipLaunchKernelGGL((conv_fwd_kernel<T, K, false>), grid, dim3(64 * kWaves), 0, stream, (const T*)a.x, a.w,
                       a.bias, (T*)a.out, a.seqlen, a.dim, ngroups, ntg);
  return hipGetLastError();
}

template <typename T, int K>
hipError_t step_k(const ConvArgs& a, hipStream_t stream) {
  const int64_t n = a.batch * a.dim;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (a.silu)
    hipLaunchKernelGGL((conv_step_kernel<T, K, true>), grid, dim3(256), 0, stream, (T*)a.state, (const T*)a.x,
                       a.w, a.bias, (T*)a.out, a.batch, a.dim);
  else
    hipLaunchKernelGGL((conv_step_kernel<T, K, false>), grid, dim3(256), 0, stream, (T*)a.state, (const T*)a.x,
                       a.w, a.bias, (T*)a.out, a.batch, a.dim);
  return hipGetLastError();
}

template <int K>
hipError_t bwd_k(const ConvArgs& a, void* ws, hipStream_t stream) {
  const ConvBwdLayout l = conv_bwd_layout(a.batch, a.seqlen, a.dim, a.width);
  float* pdw = (float*)((char*)ws + l.off_dw);
  float* pdb = (float*)((char*)ws + l.off_db);
  const int64_t ngroups = (a.dim + 63) / 64;
  const int64_t ntg = (l.ntiles + kWaves - 1) / kWaves;
  const dim3 grid((unsigned)(ngroups * ntg * a.batch));
  if (a.silu)
    hipLaunchKernelGGL((conv_bwd_kernel<K, true>), grid, dim3(64 * kWaves), 0, stream, (const float*)a.x, a.w,
                       a.bias, (const float*)a.dout, (float*)a.dx, pdw, pdb, a.seqlen, a.dim, ngroups, ntg,
                       l.ntiles);
  else
    hipLaunchKernelGGL((conv_bwd_kernel<K, false>), grid, dim3(64 * kWaves), 0, stream, (const float*)a.x, a.w,
                       a.bias, (const float*)a.dout, (float*)a.dx, pdw, pdb, a.seqlen, a.dim, ngroups, ntg,
                       l.ntiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = K * a.dim;
  hipLaunchKernelGGL((conv_reduce_kernel<K>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, pdw, pdb,
                     a.dw, a.dbias, a.batch * l.ntiles, a.dim);
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_t(const ConvArgs& a, hipStream_t s) {
  switch (a.width) {
    case 1: return fwd_k<T, 1>(a, s);
    case 2: return fwd_k<T, 2>(a, s);
    case 3: return fwd_k<T, 3>(a, s);
    case 4: return fwd_k<T, 4>(a, s);
    case 5: return fwd_k<T, 5>(a, s);
    case 6: return fwd_k<T, 6>(a, s);
    case 7: return fwd_k<T, 7>(a, s);
    default: return fwd_k<T, 8>(a, s);
  }
}
template <typename T>
hipError_t step_t(const ConvArgs& a, hipStream_t s) {
  switch (a.width) {
    case 1: return step_k<T, 1>(a, s);
    case 2: return step_k<T, 2>(a, s);
    case 3: return step_k<T, 3>(a, s);
    case 4: return step_k<T, 4>(a, s);
    case 5: return step_k<T, 5>(a, s);
    case 6: return step_k<T, 6>(a, s);
    case 7: return step_k<T, 7>(a, s);
    default: return step_k<T, 8>(a, s);
  }
}

}  // namespace

ConvBwdLayout conv_bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t width) {
  ConvBwdLayout l;
  l.ntiles = (seqlen + kBwdTile - 1) / kBwdTile;
  const size_t parts = (size_t)batch * l.ntiles;
  l.off_dw = 0;
  l.off_db = (parts * width * dim * sizeof(float) + 255) & ~(size_t)255;
  l.total = (l.off_db + parts * dim * sizeof(float) + 255) & ~(size_t)255;
  return l;
}

hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t s) {
  return a.bf16 ? fwd_t<bf16_t>(a, s) : fwd_t<float>(a, s);
}
hipError_t launch_conv_step(const ConvArgs& a, hipStream_t s) {
  return a.bf16 ? step_t<bf16_t>(a, s) : step_t<float>(a, s);
}
hipError_t launch_conv_bwd(const ConvArgs& a, void* ws, hipStream_t s) {
  switch (a.width) {
    case 1: return bwd_k<1>(a, ws, s);
    case 2: return bwd_k<2>(a, ws, s);
    case 3: return bwd_k<3>(a, ws, s);
    case 4: return bwd_k<4>(a, ws, s);
    case 5: return bwd_k<5>(a, ws, s);
    case 6: return bwd_k<6>(a, ws, s);
    case 7: return bwd_k<7>(a, ws, s);
    default: return bwd_k<8>(a, ws, s);
  }
}

}  // namespace ssm
