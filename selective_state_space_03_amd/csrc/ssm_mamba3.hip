// ssm_mamba3.hip -- adjoint of the Mamba-3 projection preprocess for gfx950.
//
// Per token row (mamba3_preprocess_backward.slang, main()): RMS-norm backward of
// every B and C group, the clamped-dt gradient with its mask and a per-row dt_bias
// partial (the page's replacement of a float atomic), the heavy-tail decay-rate
// gradient with its floor mask, and the copied z / x / trap / angle gradients.  Then
// d_dt_bias as a fixed-order sum of the row partials.
//
// Work layout (our own): one 256-thread workgroup per row.  The copies are the bulk
// of the traffic and go as contiguous 256-byte wave accesses.  Each B or C group is
// one wavefront: its lanes stride over the group's elements, and the sum of squares
// and the dot product are reduced with a fixed xor butterfly, so every lane holds the
// same totals and the result does not depend on scheduling.  Heads are spread over
// the threads.
#include "ssm_device.h"
#include "ssm_mamba3.h"
#include "ssm_scan.h"

namespace ssm {
namespace {

// sum over the 64 lanes of a wavefront, the same fixed butterfly on every lane
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

struct M3Dims {
  int64_t rows, inner, state, heads, angles, bc, width;
  int64_t off_b, off_c, off_dt, off_a, off_trap, off_ang;
};

__global__ void __launch_bounds__(256)
m3_preprocess_bwd_kernel(const float* __restrict__ projected, const float* __restrict__ dt_bias,
                         const float* __restrict__ z_grad, const float* __restrict__ x_grad,
                         const float* __restrict__ b_grad, const float* __restrict__ c_grad,
                         const float* __restrict__ dt_grad, const float* __restrict__ adt_grad,
                         const float* __restrict__ trap_grad, const float* __restrict__ angle_grad,
                         float* __restrict__ out, float* __restrict__ partial, M3Dims m, float eps,
                         float dt_min, float dt_max, float a_floor, int vec4) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* __restrict__ pr = projected + row * m.width;
  float* __restrict__ gr = out + row * m.width;

  // z and x gradients, copied: 16-byte vectors when sizes and pointers allow, four per
  // thread in flight before their stores
  if (vec4) {
    const float4* __restrict__ zs = reinterpret_cast<const float4*>(z_grad + row * m.inner);
    const float4* __restrict__ xs = reinterpret_cast<const float4*>(x_grad + row * m.inner);
    float4* __restrict__ gz = reinterpret_cast<float4*>(gr);
    float4* __restrict__ gx = reinterpret_cast<float4*>(gr + m.inner);
    const int64_t n4 = m.inner >> 2;
    for (int64_t i0 = tid; i0 < n4; i0 += 512) {
      const int64_t i1 = i0 + 256;
      const bool has1 = i1 < n4;
      const float4 z0 = zs[i0], x0 = xs[i0];
      const float4 z1 = has1 ? zs[i1] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 x1 = has1 ? xs[i1] : make_float4(0.f, 0.f, 0.f, 0.f);
      gz[i0] = z0;
      gx[i0] = x0;
      if (has1) {
        gz[i1] = z1;
        gx[i1] = x1;
      }
    }
  } else {
    for (int64_t i = tid; i < m.inner; i += 256) {
      gr[i] = z_grad[row * m.inner + i];
      gr[m.inner + i] = x_grad[row * m.inner + i];
    }
  }
  // B and C groups: wave w takes groups w, w + 4, ...
  const float inv_n = 1.0f / (float)(m.state > 0 ? m.state : 1);
  for (int64_t gi = wave; gi < 2 * m.bc; gi += 4) {
    const bool is_b = gi < m.bc;
    const int64_t grp = is_b ? gi : gi - m.bc;
    const int64_t in0 = (is_b ? m.off_b : m.off_c) + grp * m.state;
    const float* __restrict__ gp = (is_b ? b_grad : c_grad) + row * m.bc * m.state + grp * m.state;
    float ss = 0.f, dot = 0.f;
    for (int64_t i = lane; i < m.state; i += 64) {
      const float v = pr[in0 + i], g = gp[i];
      ss = fmaf(v, v, ss);
      dot = fmaf(g, v, dot);
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const float inv = 1.0f / sqrtf(fmaf(ss, inv_n, eps));
    const float c = inv * inv * inv * dot * inv_n;
    for (int64_t i = lane; i < m.state; i += 64) gr[in0 + i] = fmaf(inv, gp[i], -pr[in0 + i] * c);
  }
  // per head: dt and decay-rate gradients, the trap gradient, the row partial
  for (int64_t h = tid; h < m.heads; h += 256) {
    const int64_t s = row * m.heads + h;
    const float raw_dt = pr[m.off_dt + h] + dt_bias[h];
    const float sp = softplus_f(raw_dt);
    const float dt = clamp_delta(sp, dt_min, dt_max);
    const float raw_a = pr[m.off_a + h];
    const float ht = raw_a >= 0.f ? 1.f + raw_a : 1.f / (1.f - raw_a);
    const float a_token = -fmaxf(ht, a_floor);
    const float total = fmaf(adt_grad[s], a_token, dt_grad[s]);
    // 1 - exp(-softplus(r)) is the logistic sigmoid of r, computed without cancellation
    const float rdt = total * clamp_mask(sp, dt_min, dt_max) * sigmoid_f(raw_dt);
    gr[m.off_dt + h] = rdt;
    partial[s] = rdt;
    const float dht = raw_a >= 0.f ? 1.f : 1.f / ((1.f - raw_a) * (1.f - raw_a));
    gr[m.off_a + h] = ht > a_floor ? adt_grad[s] * dt * -dht : 0.f;
    gr[m.off_trap + h] = trap_grad[s];
  }
  for (int64_t i = tid; i < m.angles; i += 256) gr[m.off_ang + i] = angle_grad[row * m.angles + i];
}

// d_dt_bias[h] = sum over rows of partial[row][h], in a fixed order and in two passes:
// chunks of kRowChunk rows are summed in ascending row order (one wavefront per
// (chunk, 64 heads), lane = head), then the chunk sums in ascending chunk order.
constexpr int kRowChunk = 64;

__global__ void __launch_bounds__(64)
m3_dt_bias_chunk_kernel(const float* __restrict__ partial, float* __restrict__ chunk_sums, int64_t rows,
                        int64_t heads) {
  const int64_t h = (int64_t)blockIdx.y * 64 + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kRowChunk;
  if (h >= heads) return;
  const int64_t n = rows - r0 < kRowChunk ? rows - r0 : kRowChunk;
  float acc = 0.f;
#pragma unroll 16
  for (int64_t i = 0; i < n; ++i) acc += partial[(r0 + i) * heads + h];  // loads independent of acc
  chunk_sums[blockIdx.x * heads + h] = acc;
}

// the chunk sums of 64 heads: 8 threads per head each add a contiguous eighth of the
// chunks in ascending order, then the 8 sums are added in ascending order
constexpr int kFinalGroups = 8;
__global__ void __launch_bounds__(64 * kFinalGroups)
m3_dt_bias_final_kernel(const float* __restrict__ chunk_sums, float* __restrict__ d_dt_bias, int64_t nchunks,
                        int64_t heads) {
  __shared__ float sums[kFinalGroups][64];
  const int o = threadIdx.x % 64, g = threadIdx.x / 64;
  const int64_t h = (int64_t)blockIdx.x * 64 + o;
  const int64_t per = (nchunks + kFinalGroups - 1) / kFinalGroups;
  const int64_t c0 = g * per, c1 = c0 + per < nchunks ? c0 + per : nchunks;
  float acc = 0.f;
  if (h < heads) {
#pragma unroll 8
    for (int64_t c = c0; c < c1; ++c) acc += chunk_sums[c * heads + h];
  }
  sums[g][o] = acc;
  __syncthreads();
  if (g == 0 && h < heads) {
    float t = sums[0][o];
#pragma unroll
    for (int q = 1; q < kFinalGroups; ++q) t += sums[q][o];
    d_dt_bias[h] = t;
  }
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }

struct Rng {
  uintptr_t lo, hi;
};
bool overlaps(Rng a, Rng b) { return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi; }
Rng span(const void* p, size_t bytes) { return Rng{(uintptr_t)p, (uintptr_t)p + (p ? bytes : 0)}; }

}  // namespace
}  // namespace ssm

extern "C" size_t ssm_mamba3_preprocess_bwd_workspace_bytes(int64_t rows, int64_t heads) {
  if (rows < 1 || heads < 1) return 0;
  const size_t nchunks = (size_t)((rows + ssm::kRowChunk - 1) / ssm::kRowChunk);
  return (nchunks * (size_t)heads * 4 + 255) & ~(size_t)255;
}

extern "C" int ssm_mamba3_preprocess_bwd(const float* projected, const float* dt_bias, const float* z_grad,
                                         const float* x_grad, const float* b_grad, const float* c_grad,
                                         const float* dt_grad, const float* adt_grad, const float* trap_grad,
                                         const float* angle_grad, float* projected_grad, float* dt_bias_partial,
                                         float* d_dt_bias, void* workspace, size_t workspace_bytes, int64_t rows,
                                         int64_t inner, int64_t state, int64_t heads, int64_t rope_angles,
                                         int64_t bc_rows, float epsilon, float dt_min, float dt_max,
                                         float a_floor, hipStream_t stream) {
  using namespace ssm;
  if (rows < 1 || inner < 0 || state < 0 || heads < 0 || rope_angles < 0 || bc_rows < 0) return SSM_ERR_DIM;
  if (bc_rows > 0 && state < 1) return SSM_ERR_DIM;
  if (rows > 0x7fffffff) return SSM_ERR_DIM;  // one workgroup per row
  const int64_t bcw = bc_rows * state;
  const int64_t width = 2 * inner + 2 * bcw + 3 * heads + rope_angles;
  if (width < 1 || width >= ((int64_t)1 << 31)) return SSM_ERR_DIM;
  // required pointers (an input of an empty part may be NULL)
  if (!projected || !projected_grad) return SSM_ERR_NULL;
  if (inner > 0 && (!z_grad || !x_grad)) return SSM_ERR_NULL;
  if (bcw > 0 && (!b_grad || !c_grad)) return SSM_ERR_NULL;
  if (heads > 0 && (!dt_bias || !dt_grad || !adt_grad || !trap_grad || !dt_bias_partial)) return SSM_ERR_NULL;
  if (rope_angles > 0 && !angle_grad) return SSM_ERR_NULL;
  if (!(epsilon >= 0.f) || epsilon > 3.0e38f) return SSM_ERR_ARG;
  if (!(dt_min >= 0.f) || !(dt_min <= dt_max) || a_floor != a_floor) return SSM_ERR_ARG;
  const size_t ws_need = ssm_mamba3_preprocess_bwd_workspace_bytes(rows, heads);
  if (d_dt_bias && heads > 0 && (!workspace || workspace_bytes < ws_need || ((uintptr_t)workspace & 255)))
    return SSM_ERR_WORKSPACE;
  const void* all[] = {projected, dt_bias, z_grad, x_grad, b_grad, c_grad, dt_grad, adt_grad, trap_grad,
                       angle_grad, projected_grad, dt_bias_partial, d_dt_bias};
  for (const void* p : all)
    if (p && !aligned4(p)) return SSM_ERR_ALIGN;
  const size_t f = 4;
  const Rng ins[] = {span(projected, rows * width * f), span(dt_bias, heads * f), span(z_grad, rows * inner * f),
                     span(x_grad, rows * inner * f), span(b_grad, rows * bcw * f), span(c_grad, rows * bcw * f),
                     span(dt_grad, rows * heads * f), span(adt_grad, rows * heads * f),
                     span(trap_grad, rows * heads * f), span(angle_grad, rows * rope_angles * f)};
  const Rng outs[] = {span(projected_grad, rows * width * f), span(dt_bias_partial, rows * heads * f),
                      span(d_dt_bias, heads * f), span(d_dt_bias ? workspace : nullptr, ws_need)};
  for (int i = 0; i < 4; ++i) {
    for (const Rng& r : ins)
      if (overlaps(outs[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }

  M3Dims m;
  m.rows = rows; m.inner = inner; m.state = state; m.heads = heads; m.angles = rope_angles; m.bc = bc_rows;
  m.width = width;
  m.off_b = 2 * inner;
  m.off_c = m.off_b + bcw;
  m.off_dt = m.off_c + bcw;
  m.off_a = m.off_dt + heads;
  m.off_trap = m.off_a + heads;
  m.off_ang = m.off_trap + heads;
  // 16-byte copies of z and x: every row's z and x parts start 16-byte aligned
  const bool vec4 = inner % 4 == 0 && width % 4 == 0 &&
                    (((uintptr_t)projected_grad | (uintptr_t)z_grad | (uintptr_t)x_grad) & 15) == 0;
  hipLaunchKernelGGL(m3_preprocess_bwd_kernel, dim3((unsigned)rows), dim3(256), 0, stream, projected, dt_bias,
                     z_grad, x_grad, b_grad, c_grad, dt_grad, adt_grad, trap_grad, angle_grad, projected_grad,
                     dt_bias_partial, m, epsilon, dt_min, dt_max, a_floor, vec4 ? 1 : 0);
  if (hipGetLastError() != hipSuccess) return SSM_ERR_HIP;
  if (d_dt_bias && heads > 0) {
    const int64_t nchunks = (rows + kRowChunk - 1) / kRowChunk;
    const unsigned hgroups = (unsigned)((heads + 63) / 64);
    float* chunk_sums = (float*)workspace;
    hipLaunchKernelGGL(m3_dt_bias_chunk_kernel, dim3((unsigned)nchunks, hgroups), dim3(64), 0, stream,
                       dt_bias_partial, chunk_sums, rows, heads);
    if (hipGetLastError() != hipSuccess) return SSM_ERR_HIP;
    hipLaunchKernelGGL(m3_dt_bias_final_kernel, dim3(hgroups), dim3(64 * kFinalGroups), 0, stream, chunk_sums,
                       d_dt_bias, nchunks, heads);
    if (hipGetLastError() != hipSuccess) return SSM_ERR_HIP;
  }
  return SSM_OK;
}
