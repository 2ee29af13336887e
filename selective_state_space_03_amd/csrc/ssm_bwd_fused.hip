// ssm_bwd_fused.hip -- backward of the selective scan for gfx950 with every wavefront
// walking its channels' whole sequence in reverse (the path for batch x channels large
// enough to fill the chip, and for short sequences).
//
// What it computes is the backward of ssm_bwd.hip (mamba-rs kernels.rs, MambaKernels:
// ssm_backward_local, ssm_reduce_d_B / _C / _D / _a_log, softplus_bwd, silu_bwd,
// gating_backward).  With a_t = exp(Delta_t A), u_t = Delta_t x_t B_t, g_t = dy_t silu(z_t)
// and G_t = dLoss/dh_t:
//   G_t = g_t C_t + a_{t+1} G_{t+1}          (G after the last step: dh_final, or 0)
//   dz_t = dy_t s_t silu'(z_t),   s_t = sum_n C_t h_t + D x_t
//   dx_t = g_t D + Delta_t sum_n G_t B_t
//   dDelta_t = sum_n A G_t a_t h_{t-1} + x_t sum_n G_t B_t,   ddelta_raw_t = dDelta_t sigmoid(r_t)
//   dB_t = sum_d G_t Delta_t x_t,   dC_t = sum_d g_t h_t
//   dA_log = A sum_{b,t} Delta_t G_t a_t h_{t-1},   dD = sum g x,   d_dt_bias = sum ddelta_raw
//   dh0 = a_0 G_0
// The forward states come from the chunk states (the state entering every 16-step
// chunk; mamba-rs kernels.rs, ssm_burnin_fwd: a multi-step forward that saves its
// activations for the backward), written by the forward or by a states-only forward
// pass that the backward runs first.
//
// Work layout: states across lanes, as in the forward: lane 16 c + n holds state n of
// channel c (4 channels per wavefront), a workgroup is 8 wavefronts = 32 consecutive
// channels of one batch element, and each wavefront walks the 16-step chunks of the
// sequence from the last.  (4-wave workgroups, two per CU, measured the same and
// double the dB / dC partials.)  Per chunk:
//   * the workgroup stages the chunk's activation rows (x, delta_raw, z, dy; 128-byte
//     rows of its 32 channels), B and C, and the chunk's start states through LDS (in
//     fp32 with 16 states and whole channel groups, as 16-byte pieces);
//   * lane 16 c + t computes the per-element values of step t of channel c once
//     (Delta, Delta x, g, the gate terms, sigmoid(r)); the state lanes get them with
//     DPP row broadcasts, each folded into the multiply that uses it (the reverse
//     broadcasts again rather than keeping 32 broadcast registers);
//   * the chunk's forward is recomputed into VGPRs (a_t and h_t of 16 steps per lane),
//     the readout s_t is summed over the row by a transpose-reduce (lane 16 c + t ends
//     with s_t), then the reverse recurrence runs over the 16 steps;
//   * sums over states (for dx and dDelta) are two more in-row transpose-reduces; the
//     dB / dC sums over channels are permlane swaps over the 4 rows, then a fixed-order
//     sum over the 8 wavefronts through LDS, written as one partial per workgroup;
//   * dA_log accumulates per lane over the whole sequence, dD and d_dt_bias per lane
//     over time and then over the row, written as one partial per batch element.
// The partials are summed in ascending order by the reduction kernels of ssm_bwd.hip.
// No atomics: every sum has a fixed order, so the results are deterministic.
#include <utility>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kFWaves = 8;               // wavefronts per workgroup
constexpr int kFCh = 4 * kFWaves;        // channels per workgroup
constexpr int kFThr = 64 * kFWaves;      // threads per workgroup
constexpr int kFT = kStateChunk;         // steps per chunk (16)
constexpr int kFA = kFCh + 1;            // LDS row stride of [step][channel] tiles
constexpr int kFBC = 20;                 // LDS row stride of the transposed B/C tiles
constexpr int kFBCPer = 2 * kFT * 16 / kFThr;  // B/C elements each thread stages per chunk
static_assert(kFThr == kFT * kFCh, "one activation element per thread and chunk");
static_assert(kFBCPer * kFThr == 2 * kFT * 16, "whole B/C elements per thread");

// Value of lane T of the row, in every lane of the row (DPP row_newbcast).  Each per-step
// value is broadcast once into a register and every use reads that register: a value
// with several uses is not folded into its consumers, and bound_ctrl spares the zero
// initialisation of the destination (every source lane exists).
template <int T> __device__ __forceinline__ float bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kDppRowBcast0 + T, 0xf, 0xf, true));
}

// forward step T of the chunk in a state lane (each broadcast has one use, so it folds
// into the multiply as a DPP operand)
template <int T>
__device__ __forceinline__ void fstep(float (&a)[kFT], float (&h)[kFT], float& hp, float dl, float dlx, float A2,
                                      const float (&bv)[kFT]) {
  a[T] = exp2_hw(bcast<T>(dl) * A2);
  h[T] = fmaf(a[T], hp, bcast<T>(dlx) * bv[T]);
  hp = h[T];
}
template <int... I>
__device__ __forceinline__ void fwd16(std::integer_sequence<int, I...>, float (&a)[kFT], float (&h)[kFT], float& hp,
                                      float dl, float dlx, float A2, const float (&bv)[kFT]) {
  (fstep<I>(a, h, hp, dl, dlx, A2, bv), ...);
}

// A copy of v that the compiler cannot identify with v, so that a broadcast of it is not
// merged with a broadcast of v (a merged broadcast has two uses and is not folded).
__device__ __forceinline__ float fresh(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// reverse step T (T = 15 .. 0): Gc enters as a_{T+1} G_{T+1} and leaves as a_T G_T.
// dl, dlx, g, g2 are the prep lane's values (g2 a fresh copy of g): every broadcast
// below has one use.
template <int T>
__device__ __forceinline__ void rstep(float& Gc, float& dA, const float (&a)[kFT], const float (&h)[kFT],
                                      float dl, float dlx, float h0c, float g, float g2, float A,
                                      const float (&bv)[kFT], const float (&cv)[kFT], float (&r1)[kFT],
                                      float (&w)[kFT], float (&pb)[kFT], float (&pc)[kFT]) {
  const float G = fmaf(bcast<T>(g), cv[T], Gc);  // dLoss/dh_T
  pc[T] = bcast<T>(g2) * h[T];                   // dC: g_T h_T
  Gc = a[T] * G;                                 // a_T G_T, carried to step T - 1
  const float t1 = Gc * (T == 0 ? h0c : h[T > 0 ? T - 1 : 0]);  // G_T a_T h_{T-1}
  dA = fmaf(bcast<T>(dl), t1, dA);               // Delta_T G_T a_T h_{T-1}
  r1[T] = A * t1;
  w[T] = G * bv[T];
  pb[T] = bcast<T>(dlx) * G;                     // dB: G_T Delta_T x_T
}
template <int... I>
__device__ __forceinline__ void rev16(std::integer_sequence<int, I...>, float& Gc, float& dA, const float (&a)[kFT],
                                      const float (&h)[kFT], float dl, float dlx, float h0c, float g, float g2,
                                      float A, const float (&bv)[kFT], const float (&cv)[kFT], float (&r1)[kFT],
                                      float (&w)[kFT], float (&pb)[kFT], float (&pc)[kFT]) {
  (rstep<15 - I>(Gc, dA, a, h, dl, dlx, h0c, g, g2, A, bv, cv, r1, w, pb, pc), ...);
}

// v[t] of every lane 16 r + n summed over the four rows r (channels): permlane swaps
// between lanes 0-31 / 32-63 and between even / odd rows.  Lane 16 r + n ends with the
// sums for steps 4 r .. 4 r + 3 of state n, in o[0..3].
__device__ __forceinline__ void rows_sum16(float (&v)[kFT], float (&o)[4]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {  // lanes 0-31 keep step k, lanes 32-63 step k + 8
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 8]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // even rows keep v[k], odd rows v[k + 4]
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 4]), false, false);
    o[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// 16-byte buffer loads and stores (range-checked like the 4-byte ones: a 16-byte piece
// lies wholly inside or wholly outside the ranges used here)
using u32x4 = unsigned int __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void buf_st4(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// 4 consecutive elements of T as one buffer access: 16 bytes of fp32 or 8 of bf16
using u32x2 = unsigned int __attribute__((ext_vector_type(2)));
template <typename T> struct Piece;
template <> struct Piece<float> {
  using type = u32x4;
  __device__ __forceinline__ static type ld(__amdgpu_buffer_rsrc_t r, uint32_t off) { return buf_ld4(r, off); }
  __device__ __forceinline__ static void st(type v, __amdgpu_buffer_rsrc_t r, uint32_t off) { buf_st4(v, r, off); }
  __device__ __forceinline__ static float get(type v, int i) { return __uint_as_float(v[i]); }
  __device__ __forceinline__ static type make(const float (&f)[4]) {
    type v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};
template <> struct Piece<bf16_t> {
  using type = u32x2;
  __device__ __forceinline__ static type ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  }
  __device__ __forceinline__ static void st(type v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
  }
  __device__ __forceinline__ static float get(type v, int i) {  // element i: the low half first
    const uint32_t w = v[i >> 1];
    return bf16_to_f32((bf16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  __device__ __forceinline__ static type make(const float (&f)[4]) {
    type v;
#pragma unroll
    for (int i = 0; i < 2; ++i) v[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
    return v;
  }
};

// VEC: 16 states and whole 32-channel groups: thread tid moves 4 consecutive channels (or
// states) of one row as one access (16 bytes of fp32, 8 of bf16), so a wavefront issues
// at most two loads and one store per chunk instead of seven loads and four stores (the
// address units serve a wide access of 64 lanes in about the time of a 4-byte one).
template <typename T, bool GATED, bool CLAMP, bool VEC>
__global__ void __launch_bounds__(kFThr)
bwd_fused_kernel(const T* __restrict__ x, const T* __restrict__ delta_raw, const T* __restrict__ z,
                 const T* __restrict__ Bm, const T* __restrict__ Cm, const T* __restrict__ dy,
                 const float* __restrict__ A_log, const float* __restrict__ D_skip, const float* __restrict__ dt_bias,
                 const float* __restrict__ cstates, const float* __restrict__ dh_final, float* __restrict__ dh0,
                 T* __restrict__ dx, T* __restrict__ ddr, T* __restrict__ dz, float* __restrict__ pdB,
                 float* __restrict__ pdC, float* __restrict__ pdA, float* __restrict__ pdD,
                 float* __restrict__ pdbias, int L, int Dm, int N, int ngroups, float dt_lo, float dt_hi) {
  // staged inputs of a chunk (buffer k & 1 for the k-th chunk walked)
  __shared__ float act[2][4][kFT][kFA];                                   // x, delta_raw, z, dy
  __shared__ __attribute__((aligned(16))) float bcT[2][2][16][kFBC];      // B, C as [state][step]
  __shared__ float hsm[2][16][kFA];                                       // chunk start states [state][channel]
  // results of a chunk (buffer by chunk parity)
  __shared__ float outs[2][3][kFT][kFA];                                  // dx, ddelta_raw, dz
  __shared__ __attribute__((aligned(16))) float red[2][kFWaves][2][kFT * 16];  // per-wave dB, dC sums

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane >> 4, li = lane & 15;
  const int b = blockIdx.x / ngroups;
  const int grp = blockIdx.x % ngroups;
  const int g0 = grp * kFCh;
  const int cw = wave * 4 + row;  // channel of this lane inside the group
  const int d = g0 + cw;
  const bool dvalid = d < Dm;
  const bool nvalid = dvalid && li < N;
  const int nch = (L + kFT - 1) / kFT;
  const int64_t row0 = (int64_t)b * L;

  // state lane (channel d, state li)
  const float alog = nvalid ? A_log[(int64_t)d * N + li] : 0.f;
  const float A = nvalid ? -expf(alog) : 0.f;
  const float A2 = A * kLog2e;
  // prep lane (channel d, step li of the chunk)
  const float bias = (dvalid && dt_bias) ? dt_bias[d] : 0.f;
  const float dsk = (dvalid && D_skip) ? D_skip[d] : 0.f;

  // cooperative loads: thread tid moves step tid / 32, channel tid % 32 of every
  // activation row; B (tid < 256) or C of step (tid & 255) / 16, state tid % 16; and the
  // start state of state tid / 32, channel tid % 32.  All through buffer resources over
  // this batch element's slices: 32-bit offsets, and reads outside (padding channels,
  // steps past the end) return 0 without a branch.
  constexpr int ES = (int)sizeof(T);
  const int ls = tid / kFCh, lc = tid % kFCh;
  const bool lcv = g0 + lc < Dm;
  const int64_t slice = (int64_t)L * Dm * ES;
  const __amdgpu_buffer_rsrc_t rx = tile_rsrc(x + row0 * Dm, slice);
  const __amdgpu_buffer_rsrc_t rr = tile_rsrc(delta_raw + row0 * Dm, slice);
  const __amdgpu_buffer_rsrc_t rz = tile_rsrc(GATED ? z + row0 * Dm : x + row0 * Dm, slice);
  const __amdgpu_buffer_rsrc_t rdy = tile_rsrc(dy + row0 * Dm, slice);
  const __amdgpu_buffer_rsrc_t rb = tile_rsrc(Bm + row0 * N, (int64_t)L * N * ES);
  const __amdgpu_buffer_rsrc_t rc = tile_rsrc(Cm + row0 * N, (int64_t)L * N * ES);
  const __amdgpu_buffer_rsrc_t rcs = tile_rsrc(cstates + (int64_t)b * nch * N * Dm, (int64_t)nch * N * Dm * 4);
  const __amdgpu_buffer_rsrc_t rdx = tile_rsrc(dx + row0 * Dm, slice);
  const __amdgpu_buffer_rsrc_t rddr = tile_rsrc(ddr + row0 * Dm, slice);
  const __amdgpu_buffer_rsrc_t rdz = tile_rsrc(GATED ? dz + row0 * Dm : dx + row0 * Dm, GATED ? slice : 0);
  const uint32_t row_bytes = (uint32_t)(Dm * ES);
  const uint32_t aoff = lcv ? (uint32_t)(ls * Dm + g0 + lc) * ES : kOutside;  // + chunk * 16 rows
  const uint32_t coff = (lcv && ls < N) ? (uint32_t)(ls * Dm + g0 + lc) * 4 : kOutside;  // + chunk * N D
  // B/C element e = tid + kFThr i of a chunk: C when e >= 256, step (e & 255) / 16, state e % 16
  uint32_t boff[kFBCPer];
#pragma unroll
  for (int i = 0; i < kFBCPer; ++i) {
    const int e = tid + kFThr * i, bs = (e & 255) >> 4, bn = e & 15;
    boff[i] = bn < N ? (uint32_t)(bs * N + bn) * ES : kOutside;  // + chunk * 16 N
  }
  uint32_t q[2][5 + kFBCPer];  // ring of two chunks: x, delta_raw, z, dy, start state, B / C
  // VEC: thread tid moves row vs, channels (or states) vc .. vc + 3 of piece vq: the
  // activation rows x, delta_raw, z, dy (vq = 0 .. 3), then the start states (vq = 0) or
  // B and C (vq = 1: threads 128-191 B, 192-255 C, step vm / 4, states 4 (vm % 4) ..)
  const int vm = tid & 127, vq = wave >> 1;
  const int vs = vm >> 3, vc = 4 * (vm & 7);
  const int bsv = (vm & 63) >> 2, bnv = 4 * (vm & 3);
  using PT = Piece<T>;
  const uint32_t vidx = (uint32_t)(vs * Dm + g0 + vc);
  const uint32_t voff = vidx * ES;                           // + chunk * 16 rows (activations)
  const uint32_t vsoff = vidx * 4;                           // + chunk * N D (fp32 states)
  const uint32_t vboff = (uint32_t)(bsv * 16 + bnv) * ES;    // + chunk * 16 N
  typename PT::type qa[2], qb[2];  // activation piece; B or C piece (waves 2, 3)
  u32x4 qs[2];                     // start-state piece (waves 0, 1)
  auto load_chunk4 = [&](int j, int slot) __attribute__((always_inline)) {
    if (j < 0) return;
    const uint32_t o = voff + (uint32_t)j * kFT * row_bytes;
    if (vq == 0) qa[slot] = PT::ld(rx, o);
    if (vq == 1) qa[slot] = PT::ld(rr, o);
    if (GATED && vq == 2) qa[slot] = PT::ld(rz, o);
    if (vq == 3) qa[slot] = PT::ld(rdy, o);
    if (vq == 0) qs[slot] = buf_ld4(rcs, vsoff + (uint32_t)(j * N * Dm * 4));
    if (wave == 2) qb[slot] = PT::ld(rb, vboff + (uint32_t)(j * kFT * N * ES));
    if (wave == 3) qb[slot] = PT::ld(rc, vboff + (uint32_t)(j * kFT * N * ES));
  };
  auto stage_chunk4 = [&](int slot, int buf) __attribute__((always_inline)) {
    if (vq != 2 || GATED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) act[buf][vq][vs][vc + i] = PT::get(qa[slot], i);
    }
    if (vq == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) hsm[buf][vs][vc + i] = __uint_as_float(qs[slot][i]);
    }
    if (vq == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) bcT[buf][wave - 2][bnv + i][bsv] = PT::get(qb[slot], i);
    }
  };
  auto load_chunk = [&](int j, int slot) __attribute__((always_inline)) {
    if (VEC) return load_chunk4(j, slot);
    if (j < 0) return;
    const uint32_t o = off_add(aoff, (uint32_t)j * kFT * row_bytes);
    q[slot][0] = buf_ld_raw<T>(rx, o);
    q[slot][1] = buf_ld_raw<T>(rr, o);
    q[slot][2] = GATED ? buf_ld_raw<T>(rz, o) : 0u;
    q[slot][3] = buf_ld_raw<T>(rdy, o);
    q[slot][4] = buf_ld_raw<float>(rcs, off_add(coff, (uint32_t)(j * N * Dm * 4)));
#pragma unroll
    for (int i = 0; i < kFBCPer; ++i) {
      const uint32_t ob = off_add(boff[i], (uint32_t)(j * kFT * N * ES));
      q[slot][5 + i] = (tid + kFThr * i) >= 256 ? buf_ld_raw<T>(rc, ob) : buf_ld_raw<T>(rb, ob);
    }
  };
  auto stage_chunk = [&](int slot, int buf) __attribute__((always_inline)) {
    if (VEC) return stage_chunk4(slot, buf);
    act[buf][0][ls][lc] = raw_f32<T>(q[slot][0]);
    act[buf][1][ls][lc] = raw_f32<T>(q[slot][1]);
    act[buf][2][ls][lc] = raw_f32<T>(q[slot][2]);
    act[buf][3][ls][lc] = raw_f32<T>(q[slot][3]);
    hsm[buf][ls][lc] = __uint_as_float(q[slot][4]);
#pragma unroll
    for (int i = 0; i < kFBCPer; ++i) {
      const int e = tid + kFThr * i;
      bcT[buf][e >= 256 ? 1 : 0][e & 15][(e & 255) >> 4] = raw_f32<T>(q[slot][5 + i]);
    }
  };

  // The results of chunk jr (after the barrier that ends its iteration): dB / dC partials
  // (the waves' sums added in wave order) and the activation gradients as 128-byte
  // rows.  Done in the next chunk's iteration, so that these LDS reads overlap that
  // chunk's arithmetic.
  auto results4 = [&](int jr) __attribute__((always_inline)) {
    const int pr = jr & 1;
    if (vq < 3) {  // dx, ddelta_raw, dz rows
      if (vq == 2 && !GATED) return;
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = outs[pr][vq][vs][vc + i];
      const typename PT::type v = PT::make(f);
      const uint32_t o = voff + (uint32_t)jr * kFT * row_bytes;  // past the end: dropped
      if (vq == 0) PT::st(v, rdx, o);
      if (vq == 1) PT::st(v, rddr, o);
      if (GATED && vq == 2) PT::st(v, rdz, o);
    } else {  // dB (threads 384-447), dC (448-511): 4 states of one step
      const int which = wave - 6, e = 4 * (vm & 63);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kFWaves; ++v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += red[pr][v][which][e + i];
      }
      const int tt = jr * kFT + (e >> 4);
      if (tt < L) {
        const int64_t o = (((int64_t)b * ngroups + grp) * L + tt) * 16 + (e & 15);
        const float4 v4 = make_float4(acc[0], acc[1], acc[2], acc[3]);
        if (which == 0) *(float4*)(pdB + o) = v4;
        else *(float4*)(pdC + o) = v4;
      }
    }
  };
  auto results = [&](int jr) __attribute__((always_inline)) {
    if (VEC) return results4(jr);
    const int pr = jr & 1;
#pragma unroll
    for (int i = 0; i < 512 / kFThr; ++i) {
      const int e2 = tid + kFThr * i;
      const int e = e2 & 255;  // (step, state) = (e / 16, e % 16)
      const int which = e2 >> 8;
      float acc = 0.f;
#pragma unroll
      for (int v = 0; v < kFWaves; ++v) acc += red[pr][v][which][e];
      const int tt = jr * kFT + (e >> 4), nn = e & 15;
      if (tt < L && nn < N) {
        float* dst = which ? pdC : pdB;
        dst[(((int64_t)b * ngroups + grp) * L + tt) * N + nn] = acc;
      }
    }
    const uint32_t o = off_add(aoff, (uint32_t)jr * kFT * row_bytes);  // past the end: dropped
    buf_st<T>(outs[pr][0][ls][lc], rdx, o);
    buf_st<T>(outs[pr][1][ls][lc], rddr, o);
    if (GATED) buf_st<T>(outs[pr][2][ls][lc], rdz, o);
  };

  // carried over the whole sequence
  float Gc = (nvalid && dh_final) ? dh_final[((int64_t)b * Dm + d) * N + li] : 0.f;  // a_{t+1} G_{t+1}
  float dA = 0.f;                 // state lane: sum of Delta G a h_prev
  float dD_acc = 0.f, db_acc = 0.f;  // prep lane: sums of g x and of ddelta_raw over its steps

  load_chunk(nch - 1, 0);
  load_chunk(nch - 2, 1);
  stage_chunk(0, 0);
  __syncthreads();
  // unrolled by 2 so that ring slots and LDS buffers are constants: the u-th of a pair
  // reads buffer u, stages the next chunk from slot u ^ 1 and loads into slot u
  for (int kk = 0; kk < nch; kk += 2) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = kk + u;
    if (k >= nch) break;
    const int j = nch - 1 - k;  // chunk walked in this iteration
    const int buf = u, par = j & 1;
    // ---- per-element values of step li of channel cw (prep lane)
    const int t = j * kFT + li;
    const bool tv = dvalid && t < L;
    const float xv = act[buf][0][li][cw];
    const float r = act[buf][1][li][cw] + bias;
    const float zv = act[buf][2][li][cw];
    const float dyv = tv ? act[buf][3][li][cw] : 0.f;
    const float sp = softplus_f(r);
    float dl = CLAMP ? clamp_delta(sp, dt_lo, dt_hi) : sp;
    dl = tv ? dl : 0.f;  // padded steps leave the state as it is and have no gradient
    const float dlx = dl * xv;
    const float sz = GATED ? sigmoid_f(zv) : 1.f;
    const float g = GATED ? dyv * zv * sz : dyv;
    float sr = sigmoid_f(r);
    if (CLAMP) sr *= clamp_mask(sp, dt_lo, dt_hi);

    // ---- B and C of the chunk for state li, start state of this lane
    float bv[kFT], cv[kFT];
    {
      const float* pb = &bcT[buf][0][li][0];
      const float* pc = &bcT[buf][1][li][0];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 vb = *(const float4*)(pb + 4 * i);
        const float4 vc = *(const float4*)(pc + 4 * i);
        bv[4 * i] = vb.x; bv[4 * i + 1] = vb.y; bv[4 * i + 2] = vb.z; bv[4 * i + 3] = vb.w;
        cv[4 * i] = vc.x; cv[4 * i + 1] = vc.y; cv[4 * i + 2] = vc.z; cv[4 * i + 3] = vc.w;
      }
    }
    const float hstart = hsm[buf][li][cw];

    // ---- forward of the chunk: a_t and h_t of its 16 steps
    float a[kFT], h[kFT];
    float hp = hstart;
    fwd16(std::make_integer_sequence<int, kFT>(), a, h, hp, dl, dlx, A2, bv);
    // readout s_t (lane 16 c + t), then dz
    float p[kFT];
#pragma unroll
    for (int i = 0; i < kFT; ++i) p[i] = cv[i] * h[i];
    const float s = fmaf(dsk, xv, row_transpose_sum16(p, lane));
    const float dzv = GATED ? dyv * s * sz * fmaf(zv, 1.f - sz, 1.f) : 0.f;
    // Stage the next chunk (loaded one iteration ago), load the one after it, and write
    // out the previous chunk's results (complete before the last barrier).  Placed here,
    // after the forward recompute and the readout rather than right after the barrier,
    // these memory operations overlap the other wavefront's arithmetic instead of every
    // wavefront issuing them at once: 334-340 -> 320-324 us with saved states at 4x2048x2048.
    if (j > 0) stage_chunk(u ^ 1, u ^ 1);
    load_chunk(j - 2, u);
    if (k > 0) results(j + 1);

    // ---- reverse over the chunk
    float r1[kFT], w[kFT], pbv[kFT], pcv[kFT];
    rev16(std::make_integer_sequence<int, kFT>(), Gc, dA, a, h, fresh(dl), fresh(dlx), hstart, g, fresh(g), A, bv, cv,
          r1, w, pbv, pcv);
    const float sw = row_transpose_sum16(w, lane);   // sum_n G_t B_t   (lane 16 c + t)
    const float sa = row_transpose_sum16(r1, lane);  // sum_n A G_t a_t h_{t-1}
    const float dxv = fmaf(dsk, g, dl * sw);
    const float ddl = fmaf(xv, sw, sa);
    const float ddrv = ddl * sr;
    if (tv) {
      dD_acc = fmaf(g, xv, dD_acc);
      db_acc += ddrv;
    }
    outs[par][0][li][cw] = dxv;
    outs[par][1][li][cw] = ddrv;
    if (GATED) outs[par][2][li][cw] = dzv;
    // dB, dC over the wave's 4 channels, then to LDS for the sum over the 8 waves
    float ob[4], oc[4];
    rows_sum16(pbv, ob);
    rows_sum16(pcv, oc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[par][wave][0][(4 * row + i) * 16 + li] = ob[i];
      red[par][wave][1][(4 * row + i) * 16 + li] = oc[i];
    }
    __syncthreads();

  }
  }
  __syncthreads();
  results(0);

  // ---- per-sequence results
  if (dh0 && nvalid) dh0[((int64_t)b * Dm + d) * N + li] = Gc;  // a_0 G_0
  if (nvalid) pdA[((int64_t)b * N + li) * Dm + d] = dA;        // partials [b][n][d]
  const float sD = row_sum16(dD_acc), sb = row_sum16(db_acc);
  if (li == 0 && dvalid) {
    pdD[(int64_t)b * Dm + d] = sD;
    pdbias[(int64_t)b * Dm + d] = sb;
  }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

template <typename T, bool GATED>
hipError_t launch_t(const BwdArgs& a, const float* cstates, float* pdB, float* pdC, float* pdA, float* pdD,
                    float* pdb, int ngroups, hipStream_t stream) {
  const bool clamp = a.dt_lo > 0.f || a.dt_hi < __builtin_inff();
  const dim3 grid((unsigned)(a.batch * ngroups)), blk(kFThr);
  // the wide path: 16 states, whole channel groups, 16-byte aligned arrays
  bool vec = a.dstate == 16 && a.dim % kFCh == 0;
  for (const void* p : {a.x, a.delta_raw, a.z, a.dy, (const void*)a.dx, (const void*)a.ddelta_raw, (const void*)a.dz,
                        (const void*)a.B, (const void*)a.C, (const void*)cstates, (const void*)pdB, (const void*)pdC})
    vec = vec && aligned16(p);
  auto kern = clamp ? bwd_fused_kernel<T, GATED, true, false> : bwd_fused_kernel<T, GATED, false, false>;
  if (vec) kern = clamp ? bwd_fused_kernel<T, GATED, true, true> : bwd_fused_kernel<T, GATED, false, true>;
  hipLaunchKernelGGL(kern, grid, blk, 0, stream, (const T*)a.x, (const T*)a.delta_raw, (const T*)a.z, (const T*)a.B,
                     (const T*)a.C, (const T*)a.dy, a.A_log, a.D_skip, a.dt_bias, cstates, a.dh_final, a.dh0,
                     (T*)a.dx, (T*)a.ddelta_raw, (T*)a.dz, pdB, pdC, pdA, pdD, pdb, (int)a.seqlen, (int)a.dim,
                     a.dstate, ngroups, a.dt_lo, a.dt_hi);
  return hipGetLastError();
}

}  // namespace

int64_t bwd_fused_groups(int64_t dim) { return (dim + kFCh - 1) / kFCh; }

hipError_t launch_bwd_fused(const BwdArgs& a, const float* cstates, float* pdB, float* pdC, float* pdA, float* pdD,
                            float* pdb, hipStream_t stream) {
  const int ngroups = (int)bwd_fused_groups(a.dim);
  if (a.bf16)
    return a.z ? launch_t<bf16_t, true>(a, cstates, pdB, pdC, pdA, pdD, pdb, ngroups, stream)
               : launch_t<bf16_t, false>(a, cstates, pdB, pdC, pdA, pdD, pdb, ngroups, stream);
  return a.z ? launch_t<float, true>(a, cstates, pdB, pdC, pdA, pdD, pdb, ngroups, stream)
             : launch_t<float, false>(a, cstates, pdB, pdC, pdA, pdD, pdb, ngroups, stream);
}

}  // namespace ssm
