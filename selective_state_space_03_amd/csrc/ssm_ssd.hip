// ssm_ssd.hip -- the Mamba-2 SSD chunk cumsum and its ordered backward for gfx950.
//
// What is computed (deterministic_backward.py, ordered_cumsum, and the chunk cumsum
// whose backward it reorders): per (batch, head, chunk) the clamped step sizes
// dt_out = clamp(g(dt + dt_bias), dt_min, dt_max) and their running sum times A inside
// the chunk; backward, the reverse running sum of ddA times A added to ddt_out, masked
// by the clamp and scaled by g', plus the per-(batch, chunk) partials of dA and
// d_dt_bias, which a second kernel adds in ascending (batch, chunk) order (the page's
// lexical order, with no atomics).
//
// Work layout (our own).  dt and ddt are [batch, seqlen, heads] (head fastest) while the
// chunk tensors are [batch, heads, chunks, chunk] (step fastest), so every workgroup
// transposes through LDS: one workgroup per (batch, chunk, 8 heads), 4 waves, the
// chunk walked in sub-tiles of 256 steps.  The [256 steps x 8 heads] slab of dt is
// read in 32-byte head rows into LDS; then each wave takes 2 heads and handles one
// 256-step row per head with 4 consecutive steps per lane: a sequential 4-term scan in
// the lane, a 64-lane Hillis-Steele scan of the lane totals, and the carry of the
// previous sub-tile.  Rows of the chunk tensors move as 16-byte vectors when the chunk
// width and pointers allow.  Every scan and sum has a fixed order.
#include "ssm_device.h"
#include "ssm_scan.h"
#include "ssm_ssd.h"

namespace ssm {
namespace {

constexpr int kHeads = 8;    // heads per workgroup
constexpr int kHPW = kHeads / 4;  // heads per wavefront
constexpr int kSub = 256;    // steps per sub-tile (64 lanes x 4)
constexpr int kPad = 4;      // LDS row padding (keeps 16-byte row alignment)

struct SsdDims {
  int64_t L, W, nc;
  int H;
  int softplus;
  float lo, hi;
};

__device__ __forceinline__ float g_of(float r, int softplus) { return softplus ? softplus_f(r) : r; }

// inclusive scan over the 64 lanes, in increasing lane order (fixed tree)
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}
// inclusive scan from the right (lane 63 down to lane 0)
__device__ __forceinline__ float wave_incl_rscan(float v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_down(v, d, 64);
    if (lane + d < 64) v += o;
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// 4 consecutive row entries starting at p (entries at or beyond n read as 0)
template <bool VEC>
__device__ __forceinline__ void ld4(const float* __restrict__ p, int n, float (&v)[4]) {
  if (VEC && n >= 4) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = q < n ? p[q] : 0.f;
  }
}
template <bool VEC>
__device__ __forceinline__ void st4(float* __restrict__ p, int n, const float (&v)[4]) {
  if (VEC && n >= 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < n) p[q] = v[q];
  }
}

constexpr int kStage = kSub * kHeads / 256;  // slab elements per thread

// element i of a [256 steps x 16 heads] slab (step i / 16, head i % 16) lies inside the
// chunk, the sequence and the head range
__device__ __forceinline__ bool valid(int64_t t0, int n, int h0, int i, const SsdDims& m) {
  const int r = i / kHeads, h = h0 + i % kHeads;
  return r < n && t0 + r < m.L && h < m.H;
}

// dt + dt_bias of a thread's kStage slab elements (0 outside), all loads issued first
__device__ __forceinline__ void stage_load(const float* __restrict__ dt, const float* __restrict__ dt_bias, int64_t b,
                                           int64_t t0, int n, int h0, int tid, const SsdDims& m,
                                           float (&raw)[kStage]) {
  const int h = h0 + tid % kHeads;  // the same head for every j (256 is a multiple of kHeads)
  const float bias = (dt_bias && h < m.H) ? dt_bias[h] : 0.f;
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int i = tid + 256 * j;
    raw[j] = valid(t0, n, h0, i, m) ? dt[(b * m.L + t0 + i / kHeads) * m.H + h] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kStage; ++j) raw[j] += bias;
}

template <bool VEC>
__global__ void __launch_bounds__(256)
ssd_cumsum_fwd_kernel(const float* __restrict__ dt, const float* __restrict__ A, const float* __restrict__ dt_bias,
                      float* __restrict__ dA_cs, float* __restrict__ dt_out, SsdDims m) {
  __shared__ __align__(16) float tile[kHeads][kSub + kPad];
  const int64_t bc = blockIdx.x;  // (batch, chunk), chunk fastest
  const int64_t b = bc / m.nc, c = bc - b * m.nc;
  const int h0 = blockIdx.y * kHeads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float carry[kHPW] = {};
  // A of the wave's heads, loaded with the first staging loads rather than after its barrier
  float av[kHPW];
#pragma unroll
  for (int k = 0; k < kHPW; ++k) {
    const int h = h0 + wave * kHPW + k;
    av[k] = h < m.H ? A[h] : 0.f;
  }
  for (int64_t l0 = 0; l0 < m.W; l0 += kSub) {
    const int n = (int)(m.W - l0 < kSub ? m.W - l0 : kSub);
    // stage dt_out of [n steps x 16 heads], read in 64-byte head rows; all of a
    // thread's loads are issued before any of them is used
    float raw[kStage];
    stage_load(dt, dt_bias, b, c * m.W + l0, n, h0, tid, m, raw);
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int i = tid + 256 * j, r = i / kHeads, hh = i % kHeads;
      tile[hh][r] = valid(c * m.W + l0, n, h0, i, m) ? clamp_delta(g_of(raw[j], m.softplus), m.lo, m.hi) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kHPW; ++k) {
      const int hh = wave * kHPW + k, h = h0 + hh;
      if (h >= m.H) break;  // wave-uniform
      const float a = av[k];
      const float4 q = *reinterpret_cast<const float4*>(&tile[hh][4 * lane]);
      float p[4];
      p[0] = q.x * a;
      p[1] = fmaf(q.y, a, p[0]);
      p[2] = fmaf(q.z, a, p[1]);
      p[3] = fmaf(q.w, a, p[2]);
      const float s = wave_incl_scan(p[3], lane);
      float ex = __shfl_up(s, 1, 64);
      ex = lane == 0 ? 0.f : ex;
      const float off = carry[k] + ex;
      float o[4] = {off + p[0], off + p[1], off + p[2], off + p[3]};
      float d[4] = {q.x, q.y, q.z, q.w};
      carry[k] += __shfl(s, 63, 64);
      const int64_t row = ((b * m.H + h) * m.nc + c) * m.W + l0 + 4 * lane;
      const int nl = n - 4 * lane;
      if (nl > 0) {
        st4<VEC>(dA_cs + row, nl, o);
        st4<VEC>(dt_out + row, nl, d);
      }
    }
    __syncthreads();
  }
}

template <bool VEC>
__global__ void __launch_bounds__(256)
ssd_cumsum_bwd_kernel(const float* __restrict__ ddA, const float* __restrict__ ddt_out, const float* __restrict__ dt,
                      const float* __restrict__ A, const float* __restrict__ dt_bias, float* __restrict__ ddt,
                      float* __restrict__ part_a, float* __restrict__ part_b, SsdDims m) {
  __shared__ __align__(16) float tile[kHeads][kSub + kPad];
  const int64_t bc = blockIdx.x;
  const int64_t b = bc / m.nc, c = bc - b * m.nc;
  const int h0 = blockIdx.y * kHeads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float carry[kHPW] = {}, pa[kHPW] = {}, pb[kHPW] = {};
  // A of the wave's heads, loaded with the first staging loads rather than after its barrier
  float av[kHPW];
#pragma unroll
  for (int k = 0; k < kHPW; ++k) {
    const int h = h0 + wave * kHPW + k;
    av[k] = h < m.H ? A[h] : 0.f;
  }
  const int64_t nsub = (m.W + kSub - 1) / kSub;
  for (int64_t s_i = nsub - 1; s_i >= 0; --s_i) {  // sub-tiles from the end of the chunk
    const int64_t l0 = s_i * kSub;
    const int n = (int)(m.W - l0 < kSub ? m.W - l0 : kSub);
    // the ddA and ddt_out rows of the wave's heads, issued before the dt loads of the
    // staging below, so that both sets are in flight together (one round trip)
    const int nl = n - 4 * lane;
    float dA4s[kHPW][4], dO4s[kHPW][4];
#pragma unroll
    for (int k = 0; k < kHPW; ++k) {
      const int h = h0 + wave * kHPW + k;
      const int64_t row = ((b * m.H + h) * m.nc + c) * m.W + l0 + 4 * lane;
#pragma unroll
      for (int q = 0; q < 4; ++q) dA4s[k][q] = dO4s[k][q] = 0.f;
      if (nl > 0 && h < m.H) {
        ld4<VEC>(ddA + row, nl, dA4s[k]);
        ld4<VEC>(ddt_out + row, nl, dO4s[k]);
      }
    }
    // stage raw = dt + dt_bias of [n steps x kHeads heads]
    {
      float raw[kStage];
      stage_load(dt, dt_bias, b, c * m.W + l0, n, h0, tid, m, raw);
#pragma unroll
      for (int j = 0; j < kStage; ++j) {
        const int i = tid + 256 * j;
        tile[i % kHeads][i / kHeads] = raw[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kHPW; ++k) {
      const int hh = wave * kHPW + k, h = h0 + hh;
      if (h >= m.H) break;  // wave-uniform
      const float a = av[k];
      const float(&dA4)[4] = dA4s[k];
      const float(&dO4)[4] = dO4s[k];
      // reverse running sums: inside the lane, across lanes, then the later sub-tiles
      float r4[4];
      r4[3] = dA4[3];
      r4[2] = dA4[2] + r4[3];
      r4[1] = dA4[1] + r4[2];
      r4[0] = dA4[0] + r4[1];
      const float S = wave_incl_rscan(r4[0], lane);
      float ex = __shfl_down(S, 1, 64);
      ex = lane == 63 ? 0.f : ex;
      const float off = carry[k] + ex;
      carry[k] += __shfl(S, 0, 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int li = 4 * lane + q;
        if (li >= n) break;
        const float rev = off + r4[q];
        const int64_t t = c * m.W + l0 + li;
        if (t < m.L) {
          const float raw = tile[hh][li];
          const float gv = g_of(raw, m.softplus);
          const float v = clamp_delta(gv, m.lo, m.hi);
          pa[k] = fmaf(v, rev, pa[k]);
          const float gp = m.softplus ? sigmoid_f(raw) : 1.f;
          const float d = fmaf(a, rev, dO4[q]) * clamp_mask(gv, m.lo, m.hi) * gp;
          pb[k] += d;
          tile[hh][li] = d;
        }
      }
    }
    __syncthreads();
    // ddt of the slab, written in 64-byte head rows
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int i = tid + 256 * j;
      if (valid(c * m.W + l0, n, h0, i, m))
        ddt[(b * m.L + c * m.W + l0 + i / kHeads) * m.H + h0 + i % kHeads] = tile[i % kHeads][i / kHeads];
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kHPW; ++k) {
    const int h = h0 + wave * kHPW + k;
    if (h >= m.H) break;
    const float sa = wave_sum(pa[k]), sb = wave_sum(pb[k]);
    if (lane == 0) {
      part_a[bc * m.H + h] = sa;
      part_b[bc * m.H + h] = sb;
    }
  }
}

// dA[h], d_dt_bias[h]: the per-(batch, chunk) partials added in ascending (batch, chunk)
// order, one lane per head
__global__ void __launch_bounds__(64)
ssd_param_reduce_kernel(const float* __restrict__ part_a, const float* __restrict__ part_b, float* __restrict__ dA,
                        float* __restrict__ d_dt_bias, int64_t nbc, int H) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= H) return;
  float sa = 0.f, sb = 0.f;
#pragma unroll 8
  for (int64_t i = 0; i < nbc; ++i) {
    sa += part_a[i * H + h];
    sb += part_b[i * H + h];
  }
  dA[h] = sa;
  if (d_dt_bias) d_dt_bias[h] = sb;
}


// ---------------------------------------------------------------------------------
// SSD scan forward over chunks, on the matrix cores.
//
// One workgroup (8 waves) per (batch, head) walks the sequence in blocks of W = 64
// steps and keeps the [P = 64, N] state in MFMA accumulators, as 16 x 16 tiles of
// v_mfma_f32_16x16x4_f32 (lane l, register r of a tile holds row 4 * (l / 16) + r,
// column l % 16; the A operand of a lane is row l % 16, column l / 16 of the 16 x 4
// slice, the B operand row l / 16, column l % 16).  A cumsum chunk of 64 k steps is k
// consecutive blocks; a block's dA_cumsum is taken relative to the step before it
// (cs below), which leaves every decay between two of its steps unchanged.  Per block,
// with x, B, C, the state and the block's cs / dt_out staged in LDS, wave w = (row block rb = w % 4, column
// half ph = w / 4) computes the output rows 16 rb .. 16 rb + 15, columns 32 ph ..:
//   Y  = C S^T scaled by exp(cs_i)                              (K = N)
//   G  = C B^T of its rows and of the step blocks s <= its rows (split between the two
//        waves of a row block), M = G exp(cs_i - cs_s) dt_s where s <= i, else 0, to LDS
//   Y += M X over the step blocks s <= its rows, y = Y + D x, stored;
// then every wave updates its state tiles: S = exp(cs_last) S + (X exp(cs_last - cs_s)
// dt_s)^T B (K = W), computed as its transpose, so that a lane holds 4 consecutive states
// of one channel: the state is staged as 16-byte rows of [channel][state] (the layout
// that C S^T reads) and stored as 16-byte pieces.  The next chunk's x, B and C are
// loaded into registers while the matrix products run.  Sums over s and n have a fixed
// order: results are deterministic.  LDS rows are padded so that a wavefront's operand
// reads fall in distinct banks.
constexpr int kScanP = 64;  // headdim
constexpr int kScanW = 64;  // steps per block (the chunk width is a multiple of it)
constexpr int kScanThreads = 512;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Matrix-core product loops of the scan kernels, with the LDS reads of the
// next 16-wide reduction step issued before the products of the current one (the
// reads of a step are independent, so one wait covers them).  Scheduling barriers keep
// the compiler from moving the reads back next to their products.
//
// acc[j] += A T over k = 0 .. 63 for the 16 rows of A at arow (a row of 64 floats,
// scaled by `scale`) and the column tiles j of T at tcol: step kb takes k = kb + 4 lq + m
// (m = 0..3) on both operands, so A comes as one 16-byte read and T as 16 b32 reads.
// arow = the lane's row of A (row lr of the block), tcol = &T[4 lq][first column + lr].
template <int NJ, int ST_>
__device__ __forceinline__ void mm_k64(f32x4 (&acc)[NJ], const float* arow, float scale, const float* tcol, int lq) {
  f32x4 a[2];
  float bv[2][4][NJ];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if (st == 0) {
      a[0] = *(const f32x4*)&arow[4 * lq] * scale;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j) bv[0][m][j] = tcol[m * ST_ + 16 * j];
    }
    const int cur = st & 1, nxt = cur ^ 1;
    if (st < 3) {
      const int kb = 16 * (st + 1);
      a[nxt] = *(const f32x4*)&arow[kb + 4 * lq] * scale;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j) bv[nxt][m][j] = tcol[(kb + m) * ST_ + 16 * j];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = mfma4(a[cur][m], bv[cur][m][j], acc[j]);
    // the next step's LDS reads go out before this step's products
    if (st < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1 + 2 * NJ, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NJ, 0);
  }
}
// acc[q] += A B^T over the KN columns of two row-major tiles (both operands 16-byte reads):
// arow = the lane's row of A + 4 lq, brow[q] = the lane's row of B for column tile q + 4 lq
template <int KN>
__device__ __forceinline__ void mm_nt(f32x4 (&acc)[2], const float* arow, const float* brow0, const float* brow1) {
  f32x4 a[2], b0[2], b1[2];
  a[0] = *(const f32x4*)&arow[0];
  b0[0] = *(const f32x4*)&brow0[0];
  b1[0] = *(const f32x4*)&brow1[0];
#pragma unroll
  for (int st = 0; st < KN / 16; ++st) {
    const int cur = st & 1, nxt = cur ^ 1;
    if (st + 1 < KN / 16) {
      a[nxt] = *(const f32x4*)&arow[16 * (st + 1)];
      b0[nxt] = *(const f32x4*)&brow0[16 * (st + 1)];
      b1[nxt] = *(const f32x4*)&brow1[16 * (st + 1)];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[0] = mfma4(a[cur][m], b0[cur][m], acc[0]);
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[1] = mfma4(a[cur][m], b1[cur][m], acc[1]);
    // the next step's LDS reads go out before this step's products
    if (st + 1 < KN / 16) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  }
}

// C_i.B_s of every 64-step block, which all heads share (one B, C group): CB[b, blk, i, s]
// for s <= i (entries above the diagonal are not written and never read).  One
// workgroup of 8 waves per (batch, block); wave (rb, ph) takes the causal 16 x 16 blocks
// (rb, ph) and (rb, ph + 2), both operands as 16-byte reads of B and C rows straight
// from memory (rows past the end of the sequence read 0).
template <int N>
__global__ void __launch_bounds__(kScanThreads)
ssd_cb_kernel(const float* __restrict__ Bm, const float* __restrict__ Cm, float* __restrict__ CB, int64_t L,
              int64_t nblk) {
  constexpr int W = kScanW;
  const int64_t bb = blockIdx.x;  // (batch, block), block fastest
  const int64_t b = bb / nblk, blk = bb - b * nblk;
  const int64_t t0 = blk * W, nv = L - t0;
  const int nvw = nv < W ? (int)nv : W;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int ph = wave >> 2, rb = ph ? 3 - (wave & 3) : (wave & 3);
  const auto rbm = tile_rsrc(Bm + (b * L + t0) * N, (int64_t)nvw * N * 4);
  const auto rcm = tile_rsrc(Cm + (b * L + t0) * N, (int64_t)nvw * N * 4);
  float* const cbo = CB + bb * (W * W);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sb = ph + 2 * u;
    if (sb > rb) break;  // wave-uniform
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const unsigned ao = (unsigned)((16 * rb + lr) * N + 4 * lq) * 4u;
    const unsigned bo = (unsigned)((16 * sb + lr) * N + 4 * lq) * 4u;
#pragma unroll
    for (int kb = 0; kb < N; kb += 16) {
      f32x4 a, bv;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        a[m] = buf_ld<float>(rcm, ao + (unsigned)(kb + m) * 4u);
        bv[m] = buf_ld<float>(rbm, bo + (unsigned)(kb + m) * 4u);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = mfma4(a[m], bv[m], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) cbo[(16 * rb + 4 * lq + r) * W + 16 * sb + lr] = acc[r];
  }
}

// 16 bytes through a buffer resource (0 outside its range)
__device__ __forceinline__ f32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// VEC: x, B and C are 16-byte aligned (and a block's x rows span under 2 GB), and each
// thread loads the next chunk as 16-byte pieces (x: 4 channels of one step; B, C: 4
// consecutive values of the block) through buffer resources, 10 loads per thread instead
// of 40 single values and no per-load address arithmetic; B and C are then staged with
// 16-byte writes.
template <int N, bool SAVE, bool VEC>
__global__ void __launch_bounds__(kScanThreads)
ssd_chunk_scan_fwd_kernel(const float* __restrict__ x, const float* __restrict__ dt_out,
                          const float* __restrict__ dA_cs, const float* __restrict__ Bm,
                          const float* __restrict__ Cm, const float* __restrict__ Dv,
                          const float* __restrict__ h0, float* __restrict__ y, float* __restrict__ h_final,
                          float* __restrict__ block_states, const float* __restrict__ CBw, int64_t L, int H,
                          int64_t nc, int64_t cw, int64_t nct) {
  constexpr int P = kScanP, W = kScanW, T = kScanThreads;
  constexpr int SB = N + 4;  // row strides (floats) of the LDS tiles
  constexpr int SM = W + 4;
  constexpr int NT = N / 16;   // 16-column state tiles
  constexpr int TPW = NT / 2;  // state tiles per wave (32 or 16 tiles over 8 waves)
  constexpr int XL = W * P / T, BL = W * N / T;  // staged elements per thread
  __shared__ __attribute__((aligned(16))) float XT[P * SM];  // x transposed: [channel][step]
  __shared__ __attribute__((aligned(16))) float Bs[W * SB];
  __shared__ __attribute__((aligned(16))) float Cs[W * SB];
  __shared__ __attribute__((aligned(16))) float Ss[P * SB];
  __shared__ __attribute__((aligned(16))) float Ms[W * SM];
  __shared__ __attribute__((aligned(16))) float cs[W], wd[W], dts[W];

  const int64_t bh = blockIdx.x;  // (batch, head), head fastest
  const int64_t b = bh / H;
  const int h = (int)(bh - b * H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  // the two waves of a SIMD (w, w + 4) take row blocks r and 3 - r, which evens out
  // the causal work of the two phases between barriers
  const int ph = wave >> 2, rb = ph ? 3 - (wave & 3) : (wave & 3);
  const float Dh = Dv ? Dv[h] : 0.f;
  // state tiles of this wave, held transposed: tile j covers channels (pb0 + j) * 16 ..
  // and states nbw * 16 ..; lane l holds channel (pb0 + j) * 16 + l % 16 and the four
  // states nbw * 16 + 4 (l / 16) + r, r = 0..3
  const int nbw = wave % NT, pb0 = (wave / NT) * TPW;
  auto st_index = [&](int j) __attribute__((always_inline)) {
    return ((pb0 + j) * 16 + lr) * N + nbw * 16 + 4 * lq;
  };
  // block_states and h_final take 16-byte stores when 16-byte aligned (uniform)
  const bool bs16 = ((uintptr_t)block_states & 15) == 0, hf16 = ((uintptr_t)h_final & 15) == 0;

  f32x4 S[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[j][r] = h0 ? h0[bh * P * N + st_index(j) + r] : 0.f;

  // registers of the next chunk's x, B, C (element tid + T * k of each tile; VEC: piece
  // tid + T * k of 4 values)
  constexpr int XV = XL / 4, BV = BL / 4;
  static_assert(!VEC || (XV * 4 == XL && BV * 4 == BL), "whole pieces per thread");
  float rx[VEC ? 1 : XL], rbm[VEC ? 1 : BL], rcm[VEC ? 1 : BL];
  f32x4 rx4[VEC ? XV : 1], rb4[VEC ? BV : 1], rc4[VEC ? BV : 1];
  // x of step t0 + s, channel p: row (b, t0 + s, h) of x, stride H * P between steps;
  // element k of a thread is step tid / P + (T / P) k, channel tid % P.  B and C of a
  // chunk are one contiguous block of W * N values: element k is tid + T k.
  const float* const xt = x + ((b * L) * H + h) * P + (int64_t)(tid / P) * H * P + tid % P;
  const float* const bt = Bm + b * L * N + tid;
  const float* const ct = Cm + b * L * N + tid;
  const int64_t xstep = (int64_t)(T / P) * H * P;
  // x piece k of a thread: step (tid + T k) / 16, channels 4 ((tid + T k) % 16) ..; B/C piece
  // k: values 4 (tid + T k) .. of the chunk's block.  Byte offsets within the chunk are the
  // same for every chunk; a chunk's descriptors end after its last valid step, so pieces
  // of later steps (and every piece past the last chunk) read 0.
  uint32_t xo4[VEC ? XV : 1] = {};
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < XV; ++k) {
      const int i = tid + T * k;
      xo4[k] = (uint32_t)(((int64_t)(i / (P / 4)) * H * P + 4 * (i % (P / 4))) * 4);
    }
  }
  auto load_chunk_v = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * W;
    const int64_t nv = c < nc ? L - t0 : 0;  // valid steps of the chunk (may exceed W)
    const int nvw = nv < W ? (int)nv : W;
    const auto rxs = tile_rsrc(x + ((b * L + t0) * H + h) * P, nvw > 0 ? ((int64_t)(nvw - 1) * H * P + P) * 4 : 0);
    const auto rbs = tile_rsrc(Bm + (b * L + t0) * N, (int64_t)nvw * N * 4);
    const auto rcs = tile_rsrc(Cm + (b * L + t0) * N, (int64_t)nvw * N * 4);
#pragma unroll
    for (int k = 0; k < XV; ++k) rx4[k] = ld16(rxs, xo4[k]);
#pragma unroll
    for (int k = 0; k < BV; ++k) {
      const uint32_t o = (uint32_t)(tid + T * k) * 16u;
      rb4[k] = ld16(rbs, o);
      rc4[k] = ld16(rcs, o);
    }
  };
  auto load_chunk = [&](int64_t c) __attribute__((always_inline)) {
    if constexpr (VEC) {
      load_chunk_v(c);
      return;
    }
    const int64_t t0 = c * W;
    const int64_t nv = c < nc ? L - t0 : 0;  // valid steps of the chunk (may exceed W)
    const float* const xc = xt + t0 * H * P;
    const float* const bc = bt + t0 * N;
    const float* const cc = ct + t0 * N;
    if (nv >= W) {  // a whole chunk (uniform): no per-element checks
#pragma unroll
      for (int k = 0; k < XL; ++k) rx[k] = xc[k * xstep];
#pragma unroll
      for (int k = 0; k < BL; ++k) {
        rbm[k] = bc[T * k];
        rcm[k] = cc[T * k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < XL; ++k) rx[k] = (tid / P + (T / P) * k < nv) ? xc[k * xstep] : 0.f;
#pragma unroll
      for (int k = 0; k < BL; ++k) {
        const bool v = (tid + T * k) / N < nv;
        rbm[k] = v ? bc[T * k] : 0.f;
        rcm[k] = v ? cc[T * k] : 0.f;
      }
    }
  };
  load_chunk(0);

  for (int64_t c = 0; c < nc; ++c) {
    const int64_t t0 = c * W;
    // ---- stage the chunk: x rows, B and C rows, the state, cumsum and weights
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < XV; ++k) {
        const int i = tid + T * k, st = i / (P / 4), ch = 4 * (i % (P / 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) XT[(ch + j) * SM + st] = rx4[k][j];
      }
#pragma unroll
      for (int k = 0; k < BV; ++k) {
        const int e = 4 * (tid + T * k);
        *(f32x4*)&Bs[(e / N) * SB + e % N] = rb4[k];
        *(f32x4*)&Cs[(e / N) * SB + e % N] = rc4[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < XL; ++k) {
        const int i = tid + T * k;
        XT[(i % P) * SM + i / P] = rx[k];
      }
#pragma unroll
      for (int k = 0; k < BL; ++k) {
        const int i = tid + T * k;
        Bs[(i / N) * SB + i % N] = rbm[k];
        Cs[(i / N) * SB + i % N] = rcm[k];
      }
    }
    if (tid < W) {
      // block c is steps [c W, c W + W) of chunk c / (cw / W) of the cumsum; its
      // exponents are taken relative to the step before the block
      const int64_t nbc = cw / W, cc = c / nbc, o = (c - cc * nbc) * W;
      const int64_t base_i = (bh * nct + cc) * cw + o;
      const float base = o > 0 ? dA_cs[base_i - 1] : 0.f;
      const float ci = dA_cs[base_i + tid] - base, cl = dA_cs[base_i + W - 1] - base, dv = dt_out[base_i + tid];
      cs[tid] = ci;
      dts[tid] = dv;
      wd[tid] = exp2_hw((cl - ci) * kLog2e) * dv;
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      *(f32x4*)&Ss[((pb0 + j) * 16 + lr) * SB + nbw * 16 + 4 * lq] = S[j];
      // the state entering block c, [batch * heads, blocks, P, N]
      if (SAVE) {
        float* const bsp = block_states + (bh * nc + c) * P * N + st_index(j);
        if (bs16) {
          *(f32x4*)bsp = S[j];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) bsp[r] = S[j][r];
        }
      }
    }
    __syncthreads();
    // C_i.B_s of this wave's causal blocks (step blocks ph, ph + 2 that are <= rb) from
    // the shared table, in flight during C S^T
    const bool one = ph <= rb, two = ph + 2 <= rb;  // wave-uniform
    f32x4 G0 = {0.f, 0.f, 0.f, 0.f}, G1 = {0.f, 0.f, 0.f, 0.f};
    {
      const float* const cbt = CBw + ((b * nc + c) * W + 16 * rb + 4 * lq) * W + lr;
      if (one) {
#pragma unroll
        for (int r = 0; r < 4; ++r) G0[r] = cbt[r * W + ph * 16];
      }
      if (two) {
#pragma unroll
        for (int r = 0; r < 4; ++r) G1[r] = cbt[r * W + (ph + 2) * 16];
      }
    }
    load_chunk(c + 1);  // in flight during the products below (zeros past the end)

    // ---- outputs of rows 16 rb .., columns 32 ph ..: inter-chunk part
    const int i0 = 16 * rb;
    f32x4 Y[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // Products over n go in 16-wide blocks whose 4 MFMA steps take n = kb + 4 (l / 16)
    // + m (m = 0..3) on both operands: any assignment of the sum's terms to steps gives
    // the same sum, and this one lets a lane read its 4 operands as one 16-byte load.
    mm_nt<N>(Y, &Cs[(i0 + lr) * SB + 4 * lq], &Ss[(2 * ph * 16 + lr) * SB + 4 * lq],
             &Ss[((2 * ph + 1) * 16 + lr) * SB + 4 * lq]);
    float ecs[4], csr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      csr[r] = cs[i0 + 4 * lq + r];
      ecs[r] = exp2_hw(csr[r] * kLog2e);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) Y[q][r] *= ecs[r];
    // ---- masked C B^T for step blocks sb = ph, ph + 2 (those <= rb), two accumulators
    {
      if (one) {
        const int s0 = ph * 16, s1 = (ph + 2) * 16;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (u == 1 && !two) break;
          const int s = (u ? s1 : s0) + lr;
          const float css = cs[s], dv = dts[s];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = i0 + 4 * lq + r;
            const float g = u ? G1[r] : G0[r];
            // select, not a product with a mask: exp of a positive exponent may be inf
            Ms[i * SM + s] = i >= s ? g * exp2_hw((csr[r] - css) * kLog2e) * dv : 0.f;
          }
        }
      }
    }
    __syncthreads();
    // ---- Y += M X over the step blocks s <= these rows, skip term, store
    // (both operands along the steps: 16-byte reads of M's rows and of x transposed)
    for (int kb = 0; kb < 16 * (rb + 1); kb += 16) {
      const f32x4 a = *(const f32x4*)&Ms[(i0 + lr) * SM + kb + 4 * lq];
      const f32x4 x0 = *(const f32x4*)&XT[(2 * ph * 16 + lr) * SM + kb + 4 * lq];
      const f32x4 x1 = *(const f32x4*)&XT[((2 * ph + 1) * 16 + lr) * SM + kb + 4 * lq];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        Y[0] = mfma4(a[m], x0[m], Y[0]);
        Y[1] = mfma4(a[m], x1[m], Y[1]);
      }
    }
    // y[b, t0 + i, h, p] for i = i0 + 4 (l / 16) + r, p = (2 ph + q) 16 + l % 16
    float* const yrow = y + ((b * L + t0 + i0 + 4 * lq) * H + h) * P + 2 * ph * 16 + lr;
    const int64_t ystep = (int64_t)H * P;
    const bool whole = t0 + W <= L;  // uniform
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 4 * lq + r;
      if (whole || t0 + i < L) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
          yrow[r * ystep + q * 16] = fmaf(Dh, XT[((2 * ph + q) * 16 + lr) * SM + i], Y[q][r]);
      }
    }
    // ---- state: S^T = exp(cs_last) S^T + (wd B)^T X  (the step weight scales the A
    // operand, which all of the wave's tiles share)
    const float el = exp2_hw(cs[W - 1] * kLog2e);
#pragma unroll
    for (int j = 0; j < TPW; ++j) S[j] *= el;
#pragma unroll
    for (int kb = 0; kb < W; kb += 16) {
      const f32x4 w4 = *(const f32x4*)&wd[kb + 4 * lq];
      f32x4 xa[TPW];
      float bv[4];
#pragma unroll
      for (int j = 0; j < TPW; ++j) xa[j] = *(const f32x4*)&XT[((pb0 + j) * 16 + lr) * SM + kb + 4 * lq];
#pragma unroll
      for (int m = 0; m < 4; ++m) bv[m] = Bs[(kb + 4 * lq + m) * SB + nbw * 16 + lr];
      __builtin_amdgcn_sched_group_barrier(0x100, TPW + 5, 0);  // this step's reads together
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float bo = bv[m] * w4[m];
#pragma unroll
        for (int j = 0; j < TPW; ++j) S[j] = mfma4(bo, xa[j][m], S[j]);
      }
    }
    __syncthreads();  // the next chunk's staging overwrites every tile
  }
  if (h_final) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      float* const hp = h_final + bh * P * N + st_index(j);
      if (hf16) {
        *(f32x4*)hp = S[j];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) hp[r] = S[j][r];
      }
    }
  }
}


// ---------------------------------------------------------------------------------
// SSD scan backward (64-step chunks), on the matrix cores.
//
// The reverse of the forward above.  With G = dLoss/d(state leaving a chunk), S the
// state entering it (the forward's block_states), cs the chunk's dA_cumsum,
// e_i = exp(cs_i), L_is = exp(cs_i - cs_s) for s <= i, w_s = exp(cs_last - cs_s) dt_s,
// dY the chunk's dy rows, K_is = L_is C_i.B_s, Z_is = dy_i.x_s, Q = K o Z and
// V_is = L_is dt_s Z_is (s <= i), one head's share of a chunk is
//   dx_s   = w_s B_s G^T + dt_s sum_{i >= s} K_is dy_i + D dy_s
//   dB_s   = w_s x_s G  + sum_{i >= s} V_is C_i
//   dC_i   = e_i dy_i S + sum_{s <= i} V_is B_s
//   ddt_s  = sum_i Q_is + exp(cs_last - cs_s) x_s.(G B_s)
//   dcs_i  = e_i dy_i.(C_i S^T) + sum_s Q_is dt_s - dt_i sum_r Q_ri - w_i x_i.(G B_i)
//            (+ at the last step: sum_s w_s x_s.(G B_s) + e_last <G, S>)
//   G_prev = e_last G + sum_i e_i dy_i (x) C_i,    dD += sum dy x
// dcs and ddt are the gradients of dA_cumsum and dt_out, which the chunk cumsum
// backward turns into those of dt, A and dt_bias.
//
// Two kernels.  The carry kernel, one workgroup per (batch, head), runs only the G
// recurrence from the last chunk and stores the G of every chunk in a workspace, in
// the order of its accumulator fragments.  The chunk kernel, one workgroup per
// (batch, chunk, group of heads), walks its heads in ascending order: B and C are the
// same for every head, so C_i.B_s is computed once per chunk, dB and dC stay in
// accumulators across the heads (the per-head weights w and e scale the X and dY
// operands), and the V terms are summed over the heads first and multiplied by B and
// C once at the end.  dB and dC have one writer per element and no per-head copies;
// when a chunk's heads are split over several workgroups (few chunks), the groups'
// values are added in ascending group order by a second kernel, which also adds dD
// over (batch, chunk) in ascending order.  No atomics; every sum has a fixed order.
//
// Work layout of the chunk kernel (eight waves, as in the forward): wave (rb, ph) owns
// the 16 rows 16 rb .. of every [64 x *] product (as rows i or as steps s) and half of
// its columns (ph); the two waves of a SIMD take row blocks r and 3 - r.  The causal
// Z blocks of a row block are split between its two waves (step blocks ph, ph + 2).
// The row and column sums that two or four waves share go through small LDS arrays
// added in a fixed order.  G and then S pass through one LDS tile.


// the carry kernel: G of every chunk into Gbuf, dLoss/dh0 into dh0 (if given)
template <int N>
__global__ void __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(4)))
ssd_bwd_carry_kernel(const float* __restrict__ dA_cs, const float* __restrict__ Cm, const float* __restrict__ dy,
                     const float* __restrict__ dh_final, float* __restrict__ Gbuf, float* __restrict__ dh0,
                     int64_t L, int H, int64_t nc) {
  constexpr int P = kScanP, W = kScanW, T = kScanThreads;
  constexpr int SW = W + 4;    // row stride (floats) of the transposed LDS tiles
  constexpr int NT = N / 16;   // 16-column tiles of the state
  constexpr int TPW = NT / 2;  // state tiles per wave (32 or 16 tiles over 8 waves)
  constexpr int YL = W * P / T, CL = W * N / T;  // staged elements per thread
  // dy and C of the chunk transposed ([channel][step], [state][step]): both operands of
  // the update are then 16-byte reads along the steps
  __shared__ __attribute__((aligned(16))) float YT[P * SW];
  __shared__ __attribute__((aligned(16))) float CT[N * SW];
  __shared__ __attribute__((aligned(16))) float ev[W];

  const int64_t bh = blockIdx.x;  // (batch, head), head fastest
  const int64_t b = bh / H;
  const int h = (int)(bh - b * H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  // state tiles of this wave: rows (pb0 + j) 16 + 4 lq + r, columns nbw 16 + lr
  const int nbw = wave % NT, pb0 = (wave / NT) * TPW;

  f32x4 G[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      G[j][r] = dh_final ? dh_final[((bh * P) + (pb0 + j) * 16 + 4 * lq + r) * N + nbw * 16 + lr] : 0.f;

  // Thread (wave w, lane l) moves steps 8 w .. 8 w + 7 of channel l of dy and of states
  // l, l + 64 of C: each of its loads is one contiguous 256-byte row across the wave, and
  // its 8 steps go to the transposed tiles as two 16-byte writes (no bank conflicts).
  // Loads go through buffer resources with uniform bases and 32-bit lane offsets: one per
  // dy row (rows are H P values apart, too far for 32-bit offsets at many heads), one
  // per chunk of C; rows past the chunk's last valid step read 0.
  static_assert(W == 8 * (T / 64) && YL == 8 && CL == 8 * (N / 64) && P == 64, "8 steps per thread");
  const unsigned coff = (unsigned)((8 * wave) * N + lane) * 4u;
  float ry[YL], rc[CL], rcs = 0.f;
  auto load_chunk = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * W, nv = L - t0;  // valid steps (at least 1, may exceed W)
    const int nvw = nv < W ? (int)nv : W;
    const float* const yw = dy + ((b * L + t0 + 8 * wave) * H + h) * P;  // this wave's first row
    const auto rcm = tile_rsrc(Cm + (b * L + t0) * N, (int64_t)nvw * N * 4);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const auto rdy = tile_rsrc(yw + (int64_t)k * H * P, 8 * wave + k < nvw ? P * 4 : 0);
      ry[k] = buf_ld<float>(rdy, (unsigned)lane * 4u);
    }
#pragma unroll
    for (int q = 0; q < N / 64; ++q)
#pragma unroll
      for (int k = 0; k < 8; ++k) rc[8 * q + k] = buf_ld<float>(rcm, coff + (unsigned)(k * N + 64 * q) * 4u);
    if (tid < W) rcs = dA_cs[(bh * nc + c) * W + tid];
  };
  load_chunk(nc - 1);
  // fragment order: ((wave TPW + j) 64 + lane) 4 + r, P N floats per (batch, head, chunk):
  // a lane's 4 values of a tile are one 16-byte store here and one 16-byte load in the
  // chunk kernel
  float* const gfrag = Gbuf + (int64_t)wave * TPW * 256 + 4 * lane;

  for (int64_t c = nc - 1; c >= 0; --c) {
    float* const gc = gfrag + (bh * nc + c) * (int64_t)(P * N);
#pragma unroll
    for (int j = 0; j < TPW; ++j) *(f32x4*)(gc + j * 256) = G[j];
#pragma unroll
    for (int k = 0; k < 8; k += 4)
      *(f32x4*)&YT[lane * SW + 8 * wave + k] = f32x4{ry[k], ry[k + 1], ry[k + 2], ry[k + 3]};
#pragma unroll
    for (int q = 0; q < N / 64; ++q)
#pragma unroll
      for (int k = 0; k < 8; k += 4)
        *(f32x4*)&CT[(lane + 64 * q) * SW + 8 * wave + k] =
            f32x4{rc[8 * q + k], rc[8 * q + k + 1], rc[8 * q + k + 2], rc[8 * q + k + 3]};
    if (tid < W) ev[tid] = exp2_hw(rcs * kLog2e);
    __syncthreads();
    if (c > 0) load_chunk(c - 1);  // in flight during the products below

    // G = e_last G + sum_i dy_i (x) (e_i C_i)  (K = W; e scales the shared B operand)
    const float el = ev[W - 1];
#pragma unroll
    for (int j = 0; j < TPW; ++j) G[j] *= el;
    // steps k = kb + 4 lq + m (m = 0..3) of both operands from one 16-byte read each
#pragma unroll 1
    for (int kb = 0; kb < W; kb += 16) {
      const f32x4 bo = *(const f32x4*)&CT[(nbw * 16 + lr) * SW + kb + 4 * lq] *
                       *(const f32x4*)&ev[kb + 4 * lq];
      f32x4 ao[TPW];
#pragma unroll
      for (int j = 0; j < TPW; ++j) ao[j] = *(const f32x4*)&YT[((pb0 + j) * 16 + lr) * SW + kb + 4 * lq];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < TPW; ++j) G[j] = mfma4(ao[j][m], bo[m], G[j]);
    }
    __syncthreads();  // the next chunk's staging overwrites both tiles
  }
  if (dh0) {
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dh0[((bh * P) + (pb0 + j) * 16 + 4 * lq + r) * N + nbw * 16 + lr] = G[j][r];
  }
}

// the chunk kernel: dx, ddA_cumsum, ddt_out of its heads, dB and dC of its chunk summed
// over its heads (at dBo / dCo + grp * gstride), dD of each head and chunk into dDp.
// VEC: x, dy, B, C and the block states are 16-byte aligned (and a chunk's x rows span
// under 2 GB), and each thread loads them as 16-byte pieces (x, dy: 4 channels of one
// step; B, C, states: 4 consecutive values of the block), staged with 16-byte writes.  x
// and dy come through buffer resources over the head's rows of the chunk, ending after
// its last valid step, at byte offsets that are the same for every head and chunk.
// Either way a thread takes the entering state in the same pieces, so the <G, S> sums
// agree bit for bit.
template <int N, bool VEC>
__global__ void __launch_bounds__(kScanThreads)
ssd_bwd_chunk_kernel(const float* __restrict__ x, const float* __restrict__ dt_out,
                     const float* __restrict__ dA_cs, const float* __restrict__ Bm,
                     const float* __restrict__ Cm, const float* __restrict__ Dv, const float* __restrict__ dy,
                     const float* __restrict__ bstates, const float* __restrict__ Gbuf,
                     float* __restrict__ dx, float* __restrict__ ddA, float* __restrict__ ddt,
                     float* __restrict__ dBo, float* __restrict__ dCo, float* __restrict__ dDp, int64_t L, int H,
                     int64_t nc, int hpg, int ngrp, int64_t gstride) {
  constexpr int P = kScanP, W = kScanW, T = kScanThreads;
  constexpr int SX = P + 4;  // row strides (floats) of the LDS tiles
  constexpr int SB = N + 4;
  constexpr int SM = W + 4;
  constexpr int NT = N / 16;   // 16-column tiles of a [*, N] product
  constexpr int NH = NT / 2;   // ... per half
  constexpr int TPW = NT / 2;  // G fragment tiles per wave
  constexpr int XL = W * P / T, BL = W * N / T, SL = P * N / T;  // staged elements per thread
  constexpr int XV = XL / 4, BV = BL / 4, SV = SL / 4;            // ... 16-byte pieces
  static_assert(W == 64, "one lane per step of a chunk in the last phase");
  static_assert(XV * 4 == XL && BV * 4 == BL && SV * 4 == SL, "whole pieces per thread");
  __shared__ __attribute__((aligned(16))) float Xs[W * SX];
  __shared__ __attribute__((aligned(16))) float Ys[W * SX];
  __shared__ __attribute__((aligned(16))) float Bs[W * SB];
  __shared__ __attribute__((aligned(16))) float Cs[W * SB];
  __shared__ __attribute__((aligned(16))) float ST[P * SB];  // G, then the entering state
  // Ms: below the diagonal C_i.B_s (s < i, the same for every head); on and above it the
  // head's K transposed, Ms[s][i] = K_is (s <= i); at the end the V sums.  cbd: C_i.B_i.
  __shared__ __attribute__((aligned(16))) float Ms[W * SM];
  __shared__ float cbd[W];
  // per-head step values and x.(G B) partials, by head parity: the gradients of dA_cumsum
  // and dt_out of a head are formed while the next head's products run
  __shared__ float cs[2][W], dts[2][W], ev[2][W], wv[2][W];
  __shared__ float qcol[4][W];  // column sums of Q over the rows of each row block
  __shared__ float rowp[2][W];  // per half: e_i dy_i.(C_i S^T) + sum_s Q_is dt_s
  __shared__ float dwp[2][2][W];  // [parity][half]: x_s.(G B_s)
  __shared__ float red8[8];     // per-wave <G, S>
  __shared__ float redD[8];     // per-wave dy.x

  const int64_t blk = blockIdx.x;  // ((batch, chunk), head group), group fastest
  const int64_t bcn = blk / ngrp;
  const int grp = (int)(blk - bcn * ngrp);
  const int64_t b = bcn / nc, c = bcn - b * nc;
  const int hlo = grp * hpg, hhi = hlo + hpg < H ? hlo + hpg : H;
  const int64_t t0 = c * W, nv = L - t0;  // valid steps of the chunk (at least 1, may exceed W)
  const int nvw = nv < W ? (int)nv : W;   // ... within the chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lq = lane >> 4;
  const int ph = wave >> 2, rb = ph ? 3 - (wave & 3) : (wave & 3);
  const int r0 = 16 * rb;
  const int nbw = wave % NT, pb0 = (wave / NT) * TPW;

  // ---- B and C rows of the chunk (shared by every head), then C_i.B_s of this wave's
  // causal blocks into Ms below the diagonal and cbd on it
  if constexpr (VEC) {
    // piece i: values 4 i .. 4 i + 3 of the chunk's block
    const float* const bp = Bm + (b * L + t0) * N;
    const float* const cp = Cm + (b * L + t0) * N;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < BV; ++k) {
      const int e = 4 * (tid + T * k);
      const bool v = e / N < nv;
      *(f32x4*)&Bs[(e / N) * SB + e % N] = v ? *(const f32x4*)(bp + e) : zero;
      *(f32x4*)&Cs[(e / N) * SB + e % N] = v ? *(const f32x4*)(cp + e) : zero;
    }
  } else {
    const float* const bp = Bm + (b * L + t0) * N + tid;
    const float* const cp = Cm + (b * L + t0) * N + tid;
#pragma unroll 4
    for (int k = 0; k < BL; ++k) {
      const int i = tid + T * k;
      const bool v = i / N < nv;
      Bs[(i / N) * SB + i % N] = v ? bp[T * k] : 0.f;
      Cs[(i / N) * SB + i % N] = v ? cp[T * k] : 0.f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sb = ph + 2 * u;
    if (sb > rb) break;  // wave-uniform
    f32x4 KB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int kb = 0; kb < N; kb += 16) {
      const f32x4 a = *(const f32x4*)&Cs[(r0 + lr) * SB + kb + 4 * lq];
      const f32x4 bb = *(const f32x4*)&Bs[(sb * 16 + lr) * SB + kb + 4 * lq];
#pragma unroll
      for (int m = 0; m < 4; ++m) KB = mfma4(a[m], bb[m], KB);
    }
    const int s = sb * 16 + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = r0 + 4 * lq + r;
      if (s < i) Ms[i * SM + s] = KB[r];
      if (s == i) cbd[i] = KB[r];
    }
  }

  f32x4 DB[NH], DC[NH], VS[2];
#pragma unroll
  for (int j = 0; j < NH; ++j) DB[j] = DC[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  VS[0] = VS[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // x and dy of head h: element k of a thread is step tid / P + (T / P) k, channel tid % P
  const int64_t xstep = (int64_t)(T / P) * H * P;
  const int64_t xrow0 = ((b * L + t0) * H) * P + (int64_t)(tid / P) * H * P + tid % P;

  // the next head's x and dy rows, G fragment and step values, loaded one head ahead
  // (VEC: x and dy piece k of a thread is step (tid + T k) / 16, channels 4 (tid % 16) ..)
  float px[VEC ? 1 : XL], py[VEC ? 1 : XL], pc0 = 0.f, pcl = 0.f, pdt = 0.f;
  f32x4 px4[VEC ? XV : 1], py4[VEC ? XV : 1];
  f32x4 pG[TPW];
  uint32_t xo4[VEC ? XV : 1] = {};  // byte offset of x / dy piece k within a head's rows
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < XV; ++k) {
      const int i = tid + T * k;
      xo4[k] = (uint32_t)(((int64_t)(i / (P / 4)) * H * P + 4 * (i % (P / 4))) * 4);
    }
  }
  // bytes from a head's first row of the chunk to the end of its last valid row
  const int64_t xspan = ((int64_t)(nvw - 1) * H * P + P) * 4;
  auto load_head = [&](int hn) __attribute__((always_inline)) {
    const int64_t bhn = b * H + hn;
    if constexpr (VEC) {
      // pieces of steps past the end of the sequence read 0
      const auto rxs = tile_rsrc(x + ((b * L + t0) * H + hn) * P, xspan);
      const auto rys = tile_rsrc(dy + ((b * L + t0) * H + hn) * P, xspan);
#pragma unroll
      for (int k = 0; k < XV; ++k) {
        px4[k] = ld16(rxs, xo4[k]);
        py4[k] = ld16(rys, xo4[k]);
      }
    } else if (nv >= W) {  // a whole chunk (uniform): no per-element checks
      const float* const xc = x + xrow0 + (int64_t)hn * P;
      const float* const yc = dy + xrow0 + (int64_t)hn * P;
#pragma unroll
      for (int k = 0; k < XL; ++k) {
        px[k] = xc[k * xstep];
        py[k] = yc[k * xstep];
      }
    } else {
      const float* const xc = x + xrow0 + (int64_t)hn * P;
      const float* const yc = dy + xrow0 + (int64_t)hn * P;
#pragma unroll
      for (int k = 0; k < XL; ++k) {
        const bool v = tid / P + (T / P) * k < nv;
        px[k] = v ? xc[k * xstep] : 0.f;
        py[k] = v ? yc[k * xstep] : 0.f;
      }
    }
    const float* const gc = Gbuf + (bhn * nc + c) * (int64_t)(P * N) + (int64_t)wave * TPW * 256 + 4 * lane;
#pragma unroll
    for (int j = 0; j < TPW; ++j) pG[j] = *(const f32x4*)(gc + j * 256);
    if (tid < W) {
      const int64_t o = (bhn * nc + c) * W;
      pc0 = dA_cs[o + tid];
      pcl = dA_cs[o + W - 1];
      pdt = dt_out[o + tid];
    }
  };
  if (hlo < hhi) load_head(hlo);

  // ---- (f) for head hp (parity pp): gradients of dA_cumsum and dt_out, one lane per
  // step of wave 0 (W = 64), fixed-order sums (the sums over steps are butterflies).
  // Run by wave 0 after the next head's first barrier (or after the last head): the
  // next head's staging and products write the other parity's arrays, and its qcol,
  // rowp, <G, S> and dD partials only after barriers that wave 0 reaches after this.
  auto finish_head = [&](int hp, int pp) __attribute__((always_inline)) {
    const int64_t bhp = b * H + hp;
    const int sp = lane;
    const float qc = ((qcol[0][sp] + qcol[1][sp]) + qcol[2][sp]) + qcol[3][sp];
    const float dw = dwp[pp][0][sp] + dwp[pp][1][sp];
    const float g_dt = fmaf(exp2_hw((cs[pp][W - 1] - cs[pp][sp]) * kLog2e), dw, qc);
    float g_cs = (rowp[0][sp] + rowp[1][sp]) - dts[pp][sp] * qc - wv[pp][sp] * dw;
    const float tw = wave_sum64(wv[pp][sp] * dw);  // sum_s w_s x_s.(G B_s)
    if (sp == W - 1) {
      float gsum = 0.f;
      for (int kk = 0; kk < 8; ++kk) gsum += red8[kk];
      g_cs += tw + ev[pp][W - 1] * gsum;
    }
    const int64_t o = (bhp * nc + c) * W + sp;
    ddA[o] = g_cs;
    ddt[o] = g_dt;
    if (sp == 0) {
      float sD = 0.f;
      for (int kk = 0; kk < 8; ++kk) sD += redD[kk];
      dDp[bcn * H + hp] = sD;
    }
  };

  for (int h = hlo; h < hhi; ++h) {
    const int64_t bh = b * H + h;
    const int par = (h - hlo) & 1;
    // ---- (a) stage x and dy rows, G, the chunk's cumsum and weights
    if (tid < W) {
      cs[par][tid] = pc0;
      dts[par][tid] = pdt;
      ev[par][tid] = exp2_hw(pc0 * kLog2e);
      wv[par][tid] = exp2_hw((pcl - pc0) * kLog2e) * pdt;
    }
    if constexpr (VEC) {
#pragma unroll
      for (int k = 0; k < XV; ++k) {
        const int i = tid + T * k, o = (i / (P / 4)) * SX + 4 * (i % (P / 4));
        *(f32x4*)&Xs[o] = px4[k];
        *(f32x4*)&Ys[o] = py4[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < XL; ++k) {
        const int i = tid + T * k;
        Xs[(i / P) * SX + i % P] = px[k];
        Ys[(i / P) * SX + i % P] = py[k];
      }
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) ST[((pb0 + j) * 16 + 4 * lq + r) * SB + nbw * 16 + lr] = pG[j][r];
    __syncthreads();
    if (wave == 0 && h > hlo) finish_head(h - 1, par ^ 1);  // the previous head's

    // the entering state, loaded now and staged after the G products: piece k of a thread
    // is values 4 (tid + T k) .. of the block
    f32x4 rs[SV];
    {
      const float* const sc = bstates + (bh * nc + c) * (int64_t)(P * N);
#pragma unroll
      for (int k = 0; k < SV; ++k) {
        const int e = 4 * (tid + T * k);
        if constexpr (VEC) {
          rs[k] = *(const f32x4*)(sc + e);
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) rs[k][m] = sc[e + m];
        }
      }
    }

    // ---- (b) with G: B G^T (columns of half ph) and diag(w) X G (column tiles of half ph)
    f32x4 DX[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) DX[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    mm_nt<N>(DX, &Bs[(r0 + lr) * SB + 4 * lq], &ST[(2 * ph * 16 + lr) * SB + 4 * lq],
             &ST[((2 * ph + 1) * 16 + lr) * SB + 4 * lq]);
    {
      float dwq[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dwq[r] = 0.f;
#pragma unroll
        for (int q = 0; q < 2; ++q)
          dwq[r] = fmaf(DX[q][r], Xs[(r0 + 4 * lq + r) * SX + (2 * ph + q) * 16 + lr], dwq[r]);
        dwq[r] = row_sum16(dwq[r]);
      }
      if (lr == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dwp[par][ph][r0 + 4 * lq + r] = dwq[r];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ws = wv[par][r0 + 4 * lq + r];
#pragma unroll
      for (int q = 0; q < 2; ++q) DX[q][r] *= ws;
    }
    {
      const float wl = wv[par][r0 + lr];  // the weight of the A operand's row s = r0 + lr
      mm_k64<NH, SB>(DB, &Xs[(r0 + lr) * SX], wl, &ST[(4 * lq) * SB + ph * NH * 16 + lr], lq);
    }
    __syncthreads();  // ST now takes the entering state

    // ---- (c) stage S; each thread also forms its part of <G, S> from the G it replaces
    {
      float gs = 0.f;
#pragma unroll
      for (int k = 0; k < SV; ++k) {
        const int e = 4 * (tid + T * k);
        f32x4* const pst = (f32x4*)&ST[(e / N) * SB + e % N];
        const f32x4 gv = *pst;
#pragma unroll
        for (int m = 0; m < 4; ++m) gs = fmaf(gv[m], rs[k][m], gs);
        *pst = rs[k];
      }
      gs = wave_sum64(gs);
      if (lane == 0) red8[wave] = gs;
    }
    __syncthreads();
    if (h + 1 < hhi) load_head(h + 1);  // in flight during the products below

    // ---- (d) with S: diag(e) dY S (column tiles of half ph) and C S^T (columns of half ph)
    {
      const float el = ev[par][r0 + lr];  // the weight of the A operand's row i = r0 + lr
      mm_k64<NH, SB>(DC, &Ys[(r0 + lr) * SX], el, &ST[(4 * lq) * SB + ph * NH * 16 + lr], lq);
    }
    float csr[4], tot[4];
    {
      f32x4 P4[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      mm_nt<N>(P4, &Cs[(r0 + lr) * SB + 4 * lq], &ST[(2 * ph * 16 + lr) * SB + 4 * lq],
               &ST[((2 * ph + 1) * 16 + lr) * SB + 4 * lq]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        csr[r] = cs[par][r0 + 4 * lq + r];
        float rp = 0.f;
#pragma unroll
        for (int q = 0; q < 2; ++q)
          rp = fmaf(P4[q][r], Ys[(r0 + 4 * lq + r) * SX + (2 * ph + q) * 16 + lr], rp);
        tot[r] = ev[par][r0 + 4 * lq + r] * rp;
      }
    }
    // Z blocks of rows i (this row block) and step blocks sb = ph, ph + 2 (those <= rb)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int sb = ph + 2 * u;
      if (sb > rb) {
        if (lq == 0) qcol[rb][sb * 16 + lr] = 0.f;
        continue;
      }
      f32x4 ZB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int kb = 0; kb < P; kb += 16) {
        const f32x4 a = *(const f32x4*)&Ys[(r0 + lr) * SX + kb + 4 * lq];
        const f32x4 bx = *(const f32x4*)&Xs[(sb * 16 + lr) * SX + kb + 4 * lq];
#pragma unroll
        for (int m = 0; m < 4; ++m) ZB = mfma4(a[m], bx[m], ZB);
      }
      const int s = sb * 16 + lr;
      const float css = cs[par][s], dvs = dts[par][s];
      float colq = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = r0 + 4 * lq + r;
        // select, not a product with a mask: exp of a positive exponent may be inf
        const float Lis = s <= i ? exp2_hw((csr[r] - css) * kLog2e) : 0.f;
        const float cb = s < i ? Ms[i * SM + s] : (s == i ? cbd[i] : 0.f);
        const float Kv = cb * Lis;
        const float Qv = Kv * ZB[r];
        tot[r] = fmaf(Qv, dvs, tot[r]);
        colq += Qv;
        VS[u][r] = fmaf(ZB[r] * Lis, dvs, VS[u][r]);
        if (s <= i) Ms[s * SM + i] = Kv;  // K transposed, for the dx products below
      }
      colq = rows_sum4(colq);
      if (lq == 0) qcol[rb][s] = colq;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      tot[r] = row_sum16(tot[r]);
    }
    if (lr == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rowp[ph][r0 + 4 * lq + r] = tot[r];
    }

    __syncthreads();  // K of every causal block is in Ms

    // ---- (e) dx of the steps s of this row block (columns of half ph):
    // += dt_s sum_{i >= s} K_is dy_i, K^T rows from Ms (16-byte reads)
    {
      const int s = r0 + lr;
      const float dts_l = dts[par][s];
#pragma unroll
      for (int kbi = 0; kbi < 4; ++kbi) {
        if (kbi >= 4 - rb) break;  // wave-uniform: blocks rb .. 3
        const int kb = r0 + 16 * kbi;
        f32x4 a = *(const f32x4*)&Ms[s * SM + kb + 4 * lq];
        float yv[4][2];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q = 0; q < 2; ++q) yv[m][q] = Ys[(kb + 4 * lq + m) * SX + (2 * ph + q) * 16 + lr];
        __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // below the diagonal of the first block Ms holds C.B, not K: those terms are 0
          const float am = (kbi > 0 || kb + 4 * lq + m >= s) ? a[m] * dts_l : 0.f;
#pragma unroll
          for (int q = 0; q < 2; ++q) DX[q] = mfma4(am, yv[m][q], DX[q]);
        }
      }
    }
    {
      const float Dh = Dv ? Dv[h] : 0.f;
      float dD = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sr = r0 + 4 * lq + r;
        if (sr < nvw) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int p = (2 * ph + q) * 16 + lr;
            const float yv = Ys[sr * SX + p];
            dx[((b * L + t0 + sr) * H + h) * P + p] = fmaf(Dh, yv, DX[q][r]);
            dD = fmaf(yv, Xs[sr * SX + p], dD);
          }
        }
      }
      dD = wave_sum64(dD);
      if (lane == 0) redD[wave] = dD;
    }
    __syncthreads();  // qcol, rowp, dwp, <G, S> and dD partials are in LDS; tiles free

  }
  if (wave == 0 && hhi > hlo) finish_head(hhi - 1, (hhi - 1 - hlo) & 1);  // the last head's

  // ---- the V terms summed over the heads: dC_i += sum_{s <= i} V_is B_s and
  // dB_s += sum_{i >= s} V_is C_i (Ms is free: every wave passed the last barrier)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sb = ph + 2 * u;
    if (sb > rb) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) Ms[(r0 + 4 * lq + r) * SM + sb * 16 + lr] = VS[u][r];
  }
  __syncthreads();
  for (int kb = 0; kb < r0 + 16; kb += 16) {
    const f32x4 a = *(const f32x4*)&Ms[(r0 + lr) * SM + kb + 4 * lq];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int k = kb + 4 * lq + m;
#pragma unroll
      for (int j = 0; j < NH; ++j) DC[j] = mfma4(a[m], Bs[k * SB + (ph * NH + j) * 16 + lr], DC[j]);
    }
  }
  for (int kb = r0; kb < W; kb += 16) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int k = kb + 4 * lq + m;
      const float a = Ms[k * SM + r0 + lr];
#pragma unroll
      for (int j = 0; j < NH; ++j) DB[j] = mfma4(a, Cs[k * SB + (ph * NH + j) * 16 + lr], DB[j]);
    }
  }
  float* const dBg = dBo + grp * gstride;
  float* const dCg = dCo + grp * gstride;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int sr = r0 + 4 * lq + r;
    if (sr < nvw) {
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        dBg[(b * L + t0 + sr) * N + (ph * NH + j) * 16 + lr] = DB[j][r];
        dCg[(b * L + t0 + sr) * N + (ph * NH + j) * 16 + lr] = DC[j][r];
      }
    }
  }
}

// dB, dC [batch, seqlen, N]: the head groups' values added in ascending group order
// (only when a chunk's heads were split over several workgroups)
__global__ void __launch_bounds__(256)
ssd_bwd_group_sum_kernel(const float* __restrict__ dBp, const float* __restrict__ dCp, float* __restrict__ dB,
                         float* __restrict__ dC, int64_t nbln, int ngrp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nbln) return;
  float sB = 0.f, sC = 0.f;
  for (int g = 0; g < ngrp; ++g) {
    sB += dBp[g * nbln + i];
    sC += dCp[g * nbln + i];
  }
  dB[i] = sB;
  dC[i] = sC;
}

// dD [heads]: one wave per head; lane l adds the per-(batch, chunk) values l, l + 64, ..
// in ascending order, then the lanes are added by a butterfly of fixed order
__global__ void __launch_bounds__(64)
ssd_bwd_dD_kernel(const float* __restrict__ dDp, float* __restrict__ dD, int64_t nbc, int H) {
  const int h = blockIdx.x, lane = threadIdx.x;
  float s = 0.f;
  for (int64_t k = lane; k < nbc; k += 64) s += dDp[k * H + h];
  s = wave_sum(s);
  if (lane == 0) dD[h] = s;
}

struct Rng {
  uintptr_t lo, hi;
};
bool overlaps(Rng a, Rng b) { return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi; }
Rng span(const void* p, size_t bytes) { return Rng{(uintptr_t)p, (uintptr_t)p + (p ? bytes : 0)}; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// shared checks of sizes and clamp bounds; fills m
int ssd_dims(int64_t batch, int64_t seqlen, int64_t heads, int64_t chunk, int softplus, float lo, float hi,
             SsdDims& m) {
  if (batch < 1 || seqlen < 1 || heads < 1 || chunk < 1) return SSM_ERR_DIM;
  if (heads > ((int64_t)1 << 20)) return SSM_ERR_DIM;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t nc = (seqlen + chunk - 1) / chunk;
  if (seqlen >= lim || chunk >= lim || batch >= lim) return SSM_ERR_DIM;
  if ((double)batch * (double)seqlen * (double)heads >= (double)lim || batch * nc >= lim) return SSM_ERR_DIM;
  if ((double)batch * (double)heads * (double)nc * (double)chunk >= (double)lim) return SSM_ERR_DIM;
  if (!(lo >= 0.f) || !(lo <= hi)) return SSM_ERR_ARG;  // also rejects NaN bounds
  m.L = seqlen;
  m.W = chunk;
  m.nc = nc;
  m.H = (int)heads;
  m.softplus = softplus ? 1 : 0;
  m.lo = lo;
  m.hi = hi;
  return SSM_OK;
}

size_t ws_part_bytes(int64_t batch, int64_t nc, int64_t heads) {
  return ((size_t)batch * (size_t)nc * (size_t)heads * 4 + 255) & ~(size_t)255;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// heads per workgroup of the backward's chunk kernel: all of them unless there are
// at most 128 (batch, chunk) pairs, then split so that about 256 workgroups run
struct SsdBwdSplit {
  int hpg, ngrp;
};
SsdBwdSplit ssd_bwd_split(int64_t batch, int64_t nc, int64_t heads) {
  const int64_t bc = batch * nc;
  int64_t want = bc >= 256 ? 1 : 256 / bc;
  if (want > heads) want = heads;
  if (want < 1) want = 1;
  const int64_t hpg = (heads + want - 1) / want;
  return SsdBwdSplit{(int)hpg, (int)((heads + hpg - 1) / hpg)};
}

// the backward's workspace: G of every (batch, head, chunk) [P N floats each], dD per
// (batch, chunk, head), and the head groups' dB and dC when a chunk's heads are split
struct SsdBwdLayout {
  size_t g_bytes, d_bytes, p_bytes, total;
};
SsdBwdLayout ssd_bwd_layout(int64_t batch, int64_t seqlen, int64_t heads, int64_t dstate) {
  const int64_t nc = (seqlen + kScanW - 1) / kScanW;
  const SsdBwdSplit sp = ssd_bwd_split(batch, nc, heads);
  SsdBwdLayout l;
  l.g_bytes = align256((size_t)batch * heads * nc * kScanP * dstate * 4);
  l.d_bytes = align256((size_t)batch * nc * heads * 4);
  l.p_bytes = sp.ngrp > 1 ? align256((size_t)sp.ngrp * batch * seqlen * dstate * 4) : 0;
  l.total = l.g_bytes + l.d_bytes + 2 * l.p_bytes;
  return l;
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_ssd_chunk_cumsum_fwd(const float* dt, const float* A, const float* dt_bias, float* dA_cumsum,
                                        float* dt_out, int64_t batch, int64_t seqlen, int64_t heads, int64_t chunk,
                                        int dt_softplus, float dt_min, float dt_max, hipStream_t stream) {
  using namespace ssm;
  SsdDims m;
  const int st = ssd_dims(batch, seqlen, heads, chunk, dt_softplus, dt_min, dt_max, m);
  if (st != SSM_OK) return st;
  if (!dt || !A || !dA_cumsum || !dt_out) return SSM_ERR_NULL;
  const void* all[] = {dt, A, dt_bias, dA_cumsum, dt_out};
  for (const void* p : all)
    if (p && !aligned4(p)) return SSM_ERR_ALIGN;
  const size_t f = 4, nch = (size_t)batch * heads * m.nc * chunk * f;
  const Rng ins[] = {span(dt, (size_t)batch * seqlen * heads * f), span(A, heads * f), span(dt_bias, heads * f)};
  const Rng outs[] = {span(dA_cumsum, nch), span(dt_out, nch)};
  for (const Rng& o : outs)
    for (const Rng& r : ins)
      if (overlaps(o, r)) return SSM_ERR_ALIAS;
  if (overlaps(outs[0], outs[1])) return SSM_ERR_ALIAS;
  const bool vec = chunk % 4 == 0 && aligned16(dA_cumsum) && aligned16(dt_out);
  const dim3 grid((unsigned)(batch * m.nc), (unsigned)((heads + kHeads - 1) / kHeads));
  if (vec)
    hipLaunchKernelGGL(ssd_cumsum_fwd_kernel<true>, grid, dim3(256), 0, stream, dt, A, dt_bias, dA_cumsum, dt_out,
                       m);
  else
    hipLaunchKernelGGL(ssd_cumsum_fwd_kernel<false>, grid, dim3(256), 0, stream, dt, A, dt_bias, dA_cumsum, dt_out,
                       m);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" size_t ssm_ssd_chunk_cumsum_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads,
                                                          int64_t chunk) {
  if (batch < 1 || seqlen < 1 || heads < 1 || chunk < 1) return 0;
  const int64_t nc = (seqlen + chunk - 1) / chunk;
  return 2 * ssm::ws_part_bytes(batch, nc, heads);
}

extern "C" int ssm_ssd_chunk_cumsum_bwd(const float* ddA, const float* ddt_out, const float* dt, const float* A,
                                        const float* dt_bias, float* ddt, float* dA, float* d_dt_bias,
                                        void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen,
                                        int64_t heads, int64_t chunk, int dt_softplus, float dt_min, float dt_max,
                                        hipStream_t stream) {
  using namespace ssm;
  SsdDims m;
  const int st = ssd_dims(batch, seqlen, heads, chunk, dt_softplus, dt_min, dt_max, m);
  if (st != SSM_OK) return st;
  if (!ddA || !ddt_out || !dt || !A || !ddt || !dA) return SSM_ERR_NULL;
  const void* all[] = {ddA, ddt_out, dt, A, dt_bias, ddt, dA, d_dt_bias};
  for (const void* p : all)
    if (p && !aligned4(p)) return SSM_ERR_ALIGN;
  const size_t ws_need = ssm_ssd_chunk_cumsum_bwd_workspace_bytes(batch, seqlen, heads, chunk);
  if (!workspace || workspace_bytes < ws_need || ((uintptr_t)workspace & 255)) return SSM_ERR_WORKSPACE;
  const size_t f = 4, nch = (size_t)batch * heads * m.nc * chunk * f, nbl = (size_t)batch * seqlen * heads * f;
  const Rng ins[] = {span(ddA, nch), span(ddt_out, nch), span(dt, nbl), span(A, heads * f),
                     span(dt_bias, heads * f)};
  const Rng outs[] = {span(ddt, nbl), span(dA, heads * f), span(d_dt_bias, heads * f), span(workspace, ws_need)};
  for (int i = 0; i < 4; ++i) {
    for (const Rng& r : ins)
      if (overlaps(outs[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }
  float* part_a = (float*)workspace;
  float* part_b = (float*)((char*)workspace + ws_part_bytes(batch, m.nc, heads));
  const bool vec = chunk % 4 == 0 && aligned16(ddA) && aligned16(ddt_out);
  const dim3 grid((unsigned)(batch * m.nc), (unsigned)((heads + kHeads - 1) / kHeads));
  if (vec)
    hipLaunchKernelGGL(ssd_cumsum_bwd_kernel<true>, grid, dim3(256), 0, stream, ddA, ddt_out, dt, A, dt_bias, ddt,
                       part_a, part_b, m);
  else
    hipLaunchKernelGGL(ssd_cumsum_bwd_kernel<false>, grid, dim3(256), 0, stream, ddA, ddt_out, dt, A, dt_bias, ddt,
                       part_a, part_b, m);
  if (hipGetLastError() != hipSuccess) return SSM_ERR_HIP;
  hipLaunchKernelGGL(ssd_param_reduce_kernel, dim3((unsigned)((heads + 63) / 64)), dim3(64), 0, stream, part_a,
                     part_b, dA, d_dt_bias, (int64_t)(batch * m.nc), (int)heads);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" size_t ssm_ssd_chunk_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dstate) {
  if (batch < 1 || seqlen < 1 || dstate < 1) return 0;
  const int64_t nblk = (seqlen + ssm::kScanW - 1) / ssm::kScanW;
  return ssm::align256((size_t)batch * nblk * ssm::kScanW * ssm::kScanW * 4);
}

extern "C" int ssm_ssd_chunk_scan_fwd(const float* x, const float* dt_out, const float* dA_cumsum, const float* B,
                                      const float* C, const float* D, const float* h0, float* y, float* h_final,
                                      float* block_states, void* workspace, size_t workspace_bytes, int64_t batch,
                                      int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate, int64_t chunk,
                                      hipStream_t stream) {
  using namespace ssm;
  if (batch < 1 || seqlen < 1 || heads < 1 || headdim < 1 || dstate < 1 || chunk < 1) return SSM_ERR_DIM;
  const double lim = (double)((int64_t)1 << 31);
  const int64_t nc = (seqlen + chunk - 1) / chunk;
  if ((double)batch * seqlen * heads * headdim >= lim || (double)batch * heads * nc * chunk >= lim ||
      (double)batch * seqlen * dstate >= lim || (double)batch * heads * headdim * dstate >= lim ||
      (double)batch * heads >= lim)
    return SSM_ERR_DIM;
  if (headdim != kScanP || chunk % kScanW != 0 || (dstate != 64 && dstate != 128)) return SSM_ERR_UNSUPPORTED;
  if (!x || !dt_out || !dA_cumsum || !B || !C || !y) return SSM_ERR_NULL;
  const void* all[] = {x, dt_out, dA_cumsum, B, C, D, h0, y, h_final, block_states};
  for (const void* p : all)
    if (p && !aligned4(p)) return SSM_ERR_ALIGN;
  const int64_t nblk = (seqlen + kScanW - 1) / kScanW;  // 64-step blocks walked by the kernel
  if ((double)batch * heads * nblk * headdim * dstate >= lim) return SSM_ERR_DIM;
  const size_t ws_need = ssm_ssd_chunk_scan_fwd_workspace_bytes(batch, seqlen, dstate);
  if (!workspace || workspace_bytes < ws_need || ((uintptr_t)workspace & 255)) return SSM_ERR_WORKSPACE;
  const size_t f = 4, nx = (size_t)batch * seqlen * heads * headdim * f, nch = (size_t)batch * heads * nc * chunk * f;
  const size_t nbc = (size_t)batch * seqlen * dstate * f, nst = (size_t)batch * heads * headdim * dstate * f;
  const Rng ins[] = {span(x, nx), span(dt_out, nch), span(dA_cumsum, nch), span(B, nbc), span(C, nbc),
                     span(D, heads * f), span(h0, nst)};
  const Rng outs[] = {span(y, nx), span(h_final, nst), span(block_states, nst * nblk), span(workspace, ws_need)};
  for (int i = 0; i < 4; ++i) {
    for (const Rng& r : ins)
      if (overlaps(outs[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }
  float* const CBw = (float*)workspace;
  auto cbk = dstate == 128 ? ssd_cb_kernel<128> : ssd_cb_kernel<64>;
  hipLaunchKernelGGL(cbk, dim3((unsigned)(batch * nblk)), dim3(kScanThreads), 0, stream, B, C, CBw, seqlen, nblk);
  if (hipGetLastError() != hipSuccess) return SSM_ERR_HIP;
  const dim3 grid((unsigned)(batch * heads));
  // (saving the block states is a separate instantiation: the plain forward stays as lean)
  const bool vec = ((uintptr_t)x & 15) == 0 && ((uintptr_t)B & 15) == 0 && ((uintptr_t)C & 15) == 0 &&
                   (double)kScanW * heads * headdim * 4 < (double)((int64_t)1 << 31);
  auto kern = dstate == 128
                  ? (block_states ? (vec ? ssd_chunk_scan_fwd_kernel<128, true, true> : ssd_chunk_scan_fwd_kernel<128, true, false>)
                                  : (vec ? ssd_chunk_scan_fwd_kernel<128, false, true> : ssd_chunk_scan_fwd_kernel<128, false, false>))
                  : (block_states ? (vec ? ssd_chunk_scan_fwd_kernel<64, true, true> : ssd_chunk_scan_fwd_kernel<64, true, false>)
                                  : (vec ? ssd_chunk_scan_fwd_kernel<64, false, true> : ssd_chunk_scan_fwd_kernel<64, false, false>));
  hipLaunchKernelGGL(kern, grid, dim3(kScanThreads), 0, stream, x, dt_out, dA_cumsum, B, C, D, h0, y, h_final,
                     block_states, CBw, seqlen, (int)heads, nblk, chunk, nc);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

extern "C" size_t ssm_ssd_chunk_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads,
                                                        int64_t dstate) {
  if (batch < 1 || seqlen < 1 || heads < 1 || dstate < 1) return 0;
  return ssm::ssd_bwd_layout(batch, seqlen, heads, dstate).total;
}

extern "C" int ssm_ssd_chunk_scan_bwd(const float* x, const float* dt_out, const float* dA_cumsum, const float* B,
                                      const float* C, const float* D, const float* dy, const float* block_states,
                                      const float* dh_final, float* dx, float* ddA_cumsum, float* ddt_out, float* dB,
                                      float* dC, float* dD, float* dh0, void* workspace, size_t workspace_bytes,
                                      int64_t batch, int64_t seqlen, int64_t heads, int64_t headdim, int64_t dstate,
                                      int64_t chunk, hipStream_t stream) {
  using namespace ssm;
  if (batch < 1 || seqlen < 1 || heads < 1 || headdim < 1 || dstate < 1 || chunk < 1) return SSM_ERR_DIM;
  const double lim = (double)((int64_t)1 << 31);
  const int64_t nc = (seqlen + chunk - 1) / chunk;
  if ((double)batch * seqlen * heads * headdim >= lim || (double)batch * heads * nc * chunk >= lim ||
      (double)batch * seqlen * dstate * heads >= lim || (double)batch * heads * nc * headdim * dstate >= lim ||
      (double)batch * heads >= lim)
    return SSM_ERR_DIM;
  if (headdim != kScanP || chunk != kScanW || (dstate != 64 && dstate != 128)) return SSM_ERR_UNSUPPORTED;
  if (!x || !dt_out || !dA_cumsum || !B || !C || !dy || !block_states || !dx || !ddA_cumsum || !ddt_out || !dB ||
      !dC)
    return SSM_ERR_NULL;
  const void* all[] = {x, dt_out, dA_cumsum, B, C, D, dy, block_states, dh_final, dx, ddA_cumsum, ddt_out,
                       dB, dC, dD, dh0};
  for (const void* p : all)
    if (p && !aligned4(p)) return SSM_ERR_ALIGN;
  const size_t ws_need = ssm_ssd_chunk_scan_bwd_workspace_bytes(batch, seqlen, heads, dstate);
  if (!workspace || workspace_bytes < ws_need || ((uintptr_t)workspace & 255)) return SSM_ERR_WORKSPACE;
  const size_t f = 4, nx = (size_t)batch * seqlen * heads * headdim * f, nch = (size_t)batch * heads * nc * chunk * f;
  const size_t nbc = (size_t)batch * seqlen * dstate * f, nst = (size_t)batch * heads * headdim * dstate * f;
  const Rng ins[] = {span(x, nx), span(dt_out, nch), span(dA_cumsum, nch), span(B, nbc), span(C, nbc),
                     span(D, heads * f), span(dy, nx), span(block_states, nst * nc), span(dh_final, nst)};
  const Rng outs[] = {span(dx, nx), span(ddA_cumsum, nch), span(ddt_out, nch), span(dB, nbc), span(dC, nbc),
                      span(dD, heads * f), span(dh0, nst), span(workspace, ws_need)};
  constexpr int NO = sizeof(outs) / sizeof(outs[0]);
  for (int i = 0; i < NO; ++i) {
    for (const Rng& r : ins)
      if (overlaps(outs[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < NO; ++j)
      if (overlaps(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }
  const SsdBwdLayout lay = ssd_bwd_layout(batch, seqlen, heads, dstate);
  const SsdBwdSplit sp = ssd_bwd_split(batch, nc, heads);
  float* const Gbuf = (float*)workspace;
  float* const dDp = (float*)((char*)workspace + lay.g_bytes);
  float* const dBp = sp.ngrp > 1 ? (float*)((char*)workspace + lay.g_bytes + lay.d_bytes) : dB;
  float* const dCp = sp.ngrp > 1 ? (float*)((char*)workspace + lay.g_bytes + lay.d_bytes + lay.p_bytes) : dC;
  const int64_t gstride = sp.ngrp > 1 ? batch * seqlen * dstate : 0;
  auto carry = dstate == 128 ? ssd_bwd_carry_kernel<128> : ssd_bwd_carry_kernel<64>;
  hipLaunchKernelGGL(carry, dim3((unsigned)(batch * heads)), dim3(kScanThreads), 0, stream, dA_cumsum, C, dy,
                     dh_final, Gbuf, dh0, seqlen, (int)heads, nc);
  if (hipGetLastError() != hipSuccess) return SSM_ERR_HIP;
  // (the wide path addresses a chunk's x and dy rows with 32-bit byte offsets)
  const bool vec = aligned16(x) && aligned16(dy) && aligned16(B) && aligned16(C) && aligned16(block_states) &&
                   (double)kScanW * heads * headdim * 4 < (double)((int64_t)1 << 31);
  auto chunk_k = dstate == 128 ? (vec ? ssd_bwd_chunk_kernel<128, true> : ssd_bwd_chunk_kernel<128, false>)
                               : (vec ? ssd_bwd_chunk_kernel<64, true> : ssd_bwd_chunk_kernel<64, false>);
  hipLaunchKernelGGL(chunk_k, dim3((unsigned)(batch * nc * sp.ngrp)), dim3(kScanThreads), 0, stream, x, dt_out,
                     dA_cumsum, B, C, D, dy, block_states, Gbuf, dx, ddA_cumsum, ddt_out, dBp, dCp, dDp, seqlen,
                     (int)heads, nc, sp.hpg, sp.ngrp, gstride);
  if (hipGetLastError() != hipSuccess) return SSM_ERR_HIP;
  const int64_t nbln = batch * seqlen * dstate;
  if (sp.ngrp > 1) {
    hipLaunchKernelGGL(ssd_bwd_group_sum_kernel, dim3((unsigned)((nbln + 255) / 256)), dim3(256), 0, stream, dBp,
                       dCp, dB, dC, nbln, sp.ngrp);
    if (hipGetLastError() != hipSuccess) return SSM_ERR_HIP;
  }
  if (dD)
    hipLaunchKernelGGL(ssd_bwd_dD_kernel, dim3((unsigned)heads), dim3(64), 0, stream, dDp, dD, batch * nc,
                       (int)heads);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}
