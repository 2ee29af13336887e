// ssm_conv1d.hip -- depthwise causal conv1d (+ optional SiLU) for gfx950: the
// step before the selective scan in a Mamba block (mamba-rs kernels.rs, MambaKernels
// conv1d fields: conv1d_step_fwd, the one-step decode conv with SiLU;
// conv1d_burnin_fwd, the multi-step forward; conv1d_step_bwd / conv1d_burnin_bwd).
//   p[b,t,d] = sum_{k<K} w[d,k] x[b,t-(K-1)+k,d] + bias[d]   (no history before t = 0)
//   out      = silu(p) or p
// The weight and bias gradients are fixed-order sums of per-(batch, time segment)
// partials, added in lexical order (deterministic_backward.py, ordered_conv: per-batch
// partials summed in batch order, no atomics).
//
// All three kernels are HBM streams: lane = channel (two neighbouring channels per
// lane in the forward when d_inner is even), so every load and store of a [B, L, D]
// row is one contiguous segment per wavefront,
// and each lane walks a tile of TL time steps keeping the K-tap window in registers
// (the halo of K-1 rows per tile is the only re-read).  All loads of a tile are
// issued before any arithmetic.
#include <atomic>

#include "ssm_device.h"
#include "ssm_internal.h"

// Fixed scratch of the no-allocation backward (ssm_conv1d_bwd_noalloc): the per-(batch,
// segment) weight and bias partials live here instead of in a caller workspace.  Every
// GPU the library runs on holds its own copy for the life of the process.  In host code
// the name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns, cached per device by ssm::conv_scratch() below.
static __device__ __align__(256) unsigned char scratch[ssm::kConvScratchBytes];

namespace ssm {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

constexpr int kFwdTile = 32;  // time steps per lane in the forward
constexpr int kBwdTile = 16;  // time steps per lane in the backward
constexpr int kWaves = 4;     // wavefronts per workgroup, one time tile each

// V neighbouring channels per lane in one access: 2 or 4 elements of T
template <typename T, int V> struct vec_io;
template <> struct vec_io<float, 2> {
  __device__ __forceinline__ static void ld(const float* p, int64_t i, float* o) {
    const float2 q = *reinterpret_cast<const float2*>(p + i);
    o[0] = q.x; o[1] = q.y;
  }
  __device__ __forceinline__ static void st(float* p, int64_t i, const float* o) {
    *reinterpret_cast<float2*>(p + i) = make_float2(o[0], o[1]);
  }
};
template <> struct vec_io<bf16_t, 4> {
  __device__ __forceinline__ static void ld(const bf16_t* p, int64_t i, float* o) {
    const uint2 u = *reinterpret_cast<const uint2*>(p + i);
    o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
    o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
  }
  __device__ __forceinline__ static void st(bf16_t* p, int64_t i, const float* o) {
    *reinterpret_cast<uint2*>(p + i) =
        make_uint2((uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16),
                   (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16));
  }
};
// V channels per lane: 1, or an 8-byte access (2 fp32 / 4 bf16) when d_inner is a
// multiple of V and the rows are aligned for it
template <typename T, int K, bool SILU, int V>
__global__ void __launch_bounds__(64 * kWaves)
conv_fwd_kernel(const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
                T* __restrict__ out, int64_t L, int64_t Dm, int64_t ngroups, int64_t ntg) {
  constexpr int TL = kFwdTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // block -> (b, time group, channel group), channel groups fastest
  const int64_t grp = blockIdx.x % ngroups;
  const int64_t r = blockIdx.x / ngroups;
  const int64_t tg = r % ntg, b = r / ntg;
  const int64_t d = (grp * 64 + lane) * V;
  const int64_t t0 = (tg * kWaves + wave) * TL;
  if (d >= Dm || t0 >= L) return;  // no barriers in this kernel (Dm is a multiple of V)
  float wk[V][K], bs[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) wk[v][k] = w[(d + v) * K + k];
    bs[v] = bias ? bias[d + v] : 0.f;
  }
  // x[t0-K+1 .. t0+TL-1], zero before t = 0 and past the end.  Four bf16 channels stay
  // as their raw 8 bytes until used (half the registers of fp32 values), so a lane can
  // walk as many steps as in fp32; a K-row window of converted values slides along.
  constexpr bool RAW = V == 4;
  float xr[RAW ? 1 : TL + K - 1][V];
  uint2 xq[RAW ? TL + K - 1 : 1];
#pragma unroll
  for (int i = 0; i < TL + K - 1; ++i) {
    const int64_t t = t0 - (K - 1) + i;
    const bool in = t >= 0 && t < L;
    if constexpr (RAW) {
      xq[i] = in ? *reinterpret_cast<const uint2*>(x + (b * L + t) * Dm + d) : make_uint2(0u, 0u);
    } else if constexpr (V > 1) {
      if (in) {
        vec_io<T, V>::ld(x, (b * L + t) * Dm + d, xr[i]);
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v) xr[i][v] = 0.f;
      }
    } else {
      xr[i][0] = in ? io<T>::ld(x, (b * L + t) * Dm + d) : 0.f;
    }
  }
  auto row = [&](int i, int v) __attribute__((always_inline)) -> float {
    if constexpr (RAW) {
      const uint32_t u = (v < 2) ? xq[i].x : xq[i].y;
      return __uint_as_float((v & 1) ? (u & 0xffff0000u) : (u << 16));
    } else {
      return xr[i][v];
    }
  };
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    float o[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float p = bs[v];
#pragma unroll
      for (int k = 0; k < K; ++k) p = fmaf(wk[v][k], row(i + k, v), p);
      o[v] = SILU ? silu_f(p) : p;
    }
    if (t0 + i < L) {
      if constexpr (V > 1) vec_io<T, V>::st(out, (b * L + t0 + i) * Dm + d, o);
      else io<T>::st(out, (b * L + t0 + i) * Dm + d, o[0]);
    }
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

// backward of one (b, time segment, channel group): each wave walks its time tiles of
// the segment in ascending order, writes dx, and accumulates the tile's
// dw[k] = sum_t dp[t] x[t-K+1+k] and dbias = sum_t dp[t]; the waves' sums are then
// added in wave order through LDS and stored as the segment's partial, [b][seg][k][d].
// V = 2: two neighbouring channels per lane in 8-byte accesses (d_inner even, rows
// aligned), 128 channels per workgroup; the per-channel arithmetic and sum order are
// those of V = 1.
template <int K, bool SILU, int V>
__global__ void __launch_bounds__(64 * kWaves)
conv_bwd_kernel(const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
                const float* __restrict__ dout, float* __restrict__ dx, float* __restrict__ pdw,
                float* __restrict__ pdb, int64_t L, int64_t Dm, int64_t ngroups, int64_t ntg, int64_t tgs,
                int64_t nseg) {
  constexpr int TL = kBwdTile;
  __shared__ float red[kWaves][K + 1][64 * V];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t grp = blockIdx.x % ngroups;
  const int64_t r = blockIdx.x / ngroups;
  const int64_t seg = r % nseg, b = r / nseg;
  const int64_t d = grp * 64 * V + lane * V;  // first channel of the lane
  const bool dvalid = d < Dm;                 // V = 2: Dm is even, so d + 1 < Dm too
  float wk[K][V], bs[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k][v] = dvalid ? w[(d + v) * K + k] : 0.f;
    bs[v] = (dvalid && bias) ? bias[d + v] : 0.f;
  }
  float sw[K][V], sb[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    sb[v] = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) sw[k][v] = 0.f;
  }
  auto ld = [&](const float* p, int64_t i, float (&o)[V]) __attribute__((always_inline)) {
    if (V == 2) {
      const float2 q = *reinterpret_cast<const float2*>(p + i);
      o[0] = q.x; o[V - 1] = q.y;
    } else {
      o[0] = p[i];
    }
  };
  const int64_t tg_end = (seg + 1) * tgs < ntg ? (seg + 1) * tgs : ntg;
  for (int64_t tg = seg * tgs; tg < tg_end; ++tg) {
    const int64_t t0 = (tg * kWaves + wave) * TL;
    if (!dvalid || t0 >= L) continue;  // uniform per wave; the barrier below is outside the loop
    // x[t0-K+1 .. t0+TL+K-2] and dout[t0 .. t0+TL+K-2], zero outside the sequence
    constexpr int NX = TL + 2 * (K - 1), NG = TL + K - 1;
    float xr[NX][V], gr[NG][V];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int64_t t = t0 - (K - 1) + i;
      if (t >= 0 && t < L) ld(x, (b * L + t) * Dm + d, xr[i]);
      else
#pragma unroll
        for (int v = 0; v < V; ++v) xr[i][v] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int64_t t = t0 + i;
      if (t < L) ld(dout, (b * L + t) * Dm + d, gr[i]);
      else
#pragma unroll
        for (int v = 0; v < V; ++v) gr[i][v] = 0.f;
    }
    // dp[t0 + i] for i < TL + K - 1 (dp = 0 past the end since dout = 0 there)
    float dp[NG][V];
#pragma unroll
    for (int i = 0; i < NG; ++i)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if (SILU) {
          float p = bs[v];
#pragma unroll
          for (int k = 0; k < K; ++k) p = fmaf(wk[k][v], xr[i + k][v], p);
          const float sg = sigmoid_f(p);
          dp[i][v] = gr[i][v] * sg * fmaf(p, 1.f - sg, 1.f);
        } else {
          dp[i][v] = gr[i][v];
        }
      }
#pragma unroll
    for (int i = 0; i < TL; ++i) {
      float g[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        g[v] = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) g[v] = fmaf(wk[k][v], dp[i + K - 1 - k][v], g[v]);
        // the tile's own steps only (dp of the halo belongs to the next tile)
#pragma unroll
        for (int k = 0; k < K; ++k) sw[k][v] = fmaf(dp[i][v], xr[i + k][v], sw[k][v]);
        sb[v] += dp[i][v];
      }
      if (t0 + i < L) {
        if (V == 2) *reinterpret_cast<float2*>(dx + (b * L + t0 + i) * Dm + d) = make_float2(g[0], g[V - 1]);
        else dx[(b * L + t0 + i) * Dm + d] = g[0];
      }
    }
  }
  // the waves' sums, added in wave order
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) red[wave][k][lane * V + v] = sw[k][v];
    red[wave][K][lane * V + v] = sb[v];
  }
  __syncthreads();
  if (wave == 0 && dvalid) {
    const int64_t o = (b * nseg + seg) * K;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int k = 0; k <= K; ++k) {
        float s = red[0][k][lane * V + v];
#pragma unroll
        for (int u = 1; u < kWaves; ++u) s += red[u][k][lane * V + v];
        if (k < K) pdw[(o + k) * Dm + d + v] = s; else pdb[(b * nseg + seg) * Dm + d + v] = s;
      }
  }
}

// dw[d,k] and dbias[d]: sums of the partials over (b, segment) in a fixed order.  A
// workgroup takes 32 outputs (output j < K Dm is dw's (k, d) = (j / Dm, j % Dm), the
// next Dm are dbias); each of 8 threads per output adds a contiguous eighth of the
// parts in lexical order, and the 8 sums are then added in part order.
constexpr int kRedOut = 32, kRedGroups = 8;
template <int K>
__global__ void __launch_bounds__(kRedOut * kRedGroups)
conv_reduce_kernel(const float* __restrict__ pdw, const float* __restrict__ pdb, float* __restrict__ dw,
                   float* __restrict__ dbias, int64_t nparts, int64_t Dm) {
  __shared__ float sums[kRedGroups][kRedOut];
  const int o = threadIdx.x % kRedOut, g = threadIdx.x / kRedOut;
  const int64_t j = (int64_t)blockIdx.x * kRedOut + o;
  const bool isw = j < K * Dm;
  const bool live = isw ? dw != nullptr : (j < (K + 1) * Dm && dbias != nullptr);
  const int64_t per = (nparts + kRedGroups - 1) / kRedGroups;
  const int64_t p0 = g * per, p1 = p0 + per < nparts ? p0 + per : nparts;
  float s = 0.f;
  if (live) {
    const float* const src = isw ? pdw + j : pdb + (j - K * Dm);
    const int64_t stride = isw ? K * Dm : Dm;
#pragma unroll 8
    for (int64_t p = p0; p < p1; ++p) s += src[p * stride];
  }
  sums[g][o] = s;
  __syncthreads();
  if (g == 0 && live) {
    float t = sums[0][o];
#pragma unroll
    for (int q = 1; q < kRedGroups; ++q) t += sums[q][o];
    if (isw)
      dw[(j % Dm) * K + j / Dm] = t;
    else
      dbias[j - K * Dm] = t;
  }
}

template <typename T, int K, int V>
hipError_t fwd_kv(const ConvArgs& a, hipStream_t stream) {
  constexpr int TL = kFwdTile;
  const int64_t ngroups = (a.dim + 64 * V - 1) / (64 * V);
  const int64_t ntg = (a.seqlen + TL * kWaves - 1) / (TL * kWaves);
  const dim3 grid((unsigned)(ngroups * ntg * a.batch));
  if (a.silu)
    hipLaunchKernelGGL((conv_fwd_kernel<T, K, true, V>), grid, dim3(64 * kWaves), 0, stream, (const T*)a.x, a.w,
                       a.bias, (T*)a.out, a.seqlen, a.dim, ngroups, ntg);
  else
    hipLaunchKernelGGL((conv_fwd_kernel<T, K, false, V>), grid, dim3(64 * kWaves), 0, stream, (const T*)a.x, a.w,
                       a.bias, (T*)a.out, a.seqlen, a.dim, ngroups, ntg);
  return hipGetLastError();
}

template <typename T, int K>
hipError_t fwd_k(const ConvArgs& a, hipStream_t stream) {
  // 8-byte accesses (2 fp32 or 4 bf16 channels per lane) when every row starts on
  // an 8-byte boundary
  constexpr int V = sizeof(T) == 4 ? 2 : 4;
  if (a.dim % V == 0 && (uintptr_t)a.x % 8 == 0 && (uintptr_t)a.out % 8 == 0)
    return fwd_kv<T, K, V>(a, stream);
  return fwd_kv<T, K, 1>(a, stream);
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
  // two channels per lane when d_inner is even and x, dout, dx allow 8-byte accesses
  const bool v2 = a.dim % 2 == 0 && ((uintptr_t)a.x & 7) == 0 && ((uintptr_t)a.dout & 7) == 0 &&
                  ((uintptr_t)a.dx & 7) == 0;
  const int64_t ngroups = v2 ? (a.dim + 127) / 128 : (a.dim + 63) / 64;
  const dim3 grid((unsigned)(ngroups * l.nseg * a.batch));
  auto kern = a.silu ? (v2 ? conv_bwd_kernel<K, true, 2> : conv_bwd_kernel<K, true, 1>)
                     : (v2 ? conv_bwd_kernel<K, false, 2> : conv_bwd_kernel<K, false, 1>);
  hipLaunchKernelGGL(kern, grid, dim3(64 * kWaves), 0, stream, (const float*)a.x, a.w, a.bias,
                     (const float*)a.dout, (float*)a.dx, pdw, pdb, a.seqlen, a.dim, ngroups, l.ntg, l.tgs, l.nseg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (K + 1) * a.dim;
  hipLaunchKernelGGL((conv_reduce_kernel<K>), dim3((unsigned)((n + kRedOut - 1) / kRedOut)),
                     dim3(kRedOut * kRedGroups), 0, stream, pdw, pdb, a.dw, a.dbias, a.batch * l.nseg, a.dim);
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
  // time groups of kWaves tiles; a workgroup walks tgs of them (a segment), with tgs
  // chosen for about 1536 workgroups in all
  l.ntg = (seqlen + kBwdTile * kWaves - 1) / (kBwdTile * kWaves);
  const int64_t units = l.ntg * ((dim + 63) / 64) * batch;
  l.tgs = (units + 1535) / 1536;
  if (l.tgs < 1) l.tgs = 1;
  l.nseg = (l.ntg + l.tgs - 1) / l.tgs;
  const size_t parts = (size_t)batch * l.nseg;
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
// Device address of this device's scratch array: resolved with hipGetSymbolAddress
// (current device) on the first call on each device, then reused.
hipError_t conv_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // same value from any racing thread
  }
  *out = p;
  return hipSuccess;
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
