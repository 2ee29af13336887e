// ssm_device.h -- device helpers of the gfx950 selective-scan kernels.
//
// Precision policy (mamba-rs kernels.rs, MambaKernels::compile: no fast-math, because
// flushed denormals and approximate exp/sqrt break gradient flow through long
// recurrences): every kernel is built without -ffast-math, fp32 denormals stay
// enabled, and the transcendental functions below are the hardware v_exp_f32,
// v_log_f32 and v_rcp_f32 (about 1 ulp each), wrapped in formulas that keep full
// relative accuracy where the textbook form would cancel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssm {

typedef uint16_t bf16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float log2_hw(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float rcp_hw(float v) { return __builtin_amdgcn_rcpf(v); }

// softplus(r) = log(1 + exp(r)) = max(r, 0) + log1p(e), e = exp(-|r|) in (0, 1].
// log1p(e) = log(u) - c with u = fl(1 + e) and c = (u - 1) - e, the exact rounding
// error of the sum: this keeps full relative accuracy for tiny e (large |r|) with no
// branch, and never overflows.  The pages' softplus (POPCORNBENCH transcript,
// softplus device function) guards with thresholds at +-20; this form needs none.
__device__ __forceinline__ float softplus_f(float r) {
  const float e = exp2_hw(-fabsf(r) * kLog2e);
  const float u = 1.0f + e;
  const float c = (u - 1.0f) - e;
  return fmaxf(r, 0.0f) + fmaf(log2_hw(u), kLn2, -c);
}

// The optional step-size clamp (mamba3_preprocess_backward.slang clamps softplus to
// [dt_min, dt_max] and masks the gradient of the clamped steps): Delta = softplus
// clamped to [lo, hi].  lo = 0, hi = +inf is no clamp at all, since softplus >= 0.
// Written with comparisons so that a NaN stays NaN.
__device__ __forceinline__ float clamp_delta(float sp, float lo, float hi) {
  return sp < lo ? lo : (sp > hi ? hi : sp);
}
// 1 where the clamp lets the gradient through (softplus inside [lo, hi], bounds
// included), else 0
__device__ __forceinline__ float clamp_mask(float sp, float lo, float hi) {
  return (sp >= lo && sp <= hi) ? 1.f : 0.f;
}

// logistic sigmoid, the derivative of softplus (mamba3_preprocess_backward.slang writes
// it as 1 - exp(-softplus(r))).  exp2 saturates to +inf for r << 0 and rcp(inf) = 0.
__device__ __forceinline__ float sigmoid_f(float r) { return rcp_hw(1.0f + exp2_hw(-r * kLog2e)); }

// silu(z) = z * sigmoid(z)  (mamba-rs silu_fwd)
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// round-to-nearest-even fp32 -> bf16 (NaN stays NaN)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
  __device__ __forceinline__ static float ld(const float* __restrict__ p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void st(float* __restrict__ p, int64_t i, float v) { p[i] = v; }
};
template <> struct io<bf16_t> {
  __device__ __forceinline__ static float ld(const bf16_t* __restrict__ p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void st(bf16_t* __restrict__ p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Raw element bits (fp32 bits, or a bf16 value zero-extended) and their fp32 value.
// Prefetch registers hold the raw bits and convert at the value's first use, so the
// wait for a load is not pulled up to the conversion right after it.
template <typename T> __device__ __forceinline__ uint32_t ld_bits(const T* __restrict__ p, int64_t i);
template <> __device__ __forceinline__ uint32_t ld_bits<float>(const float* __restrict__ p, int64_t i) {
  return __float_as_uint(p[i]);
}
template <> __device__ __forceinline__ uint32_t ld_bits<bf16_t>(const bf16_t* __restrict__ p, int64_t i) {
  return (uint32_t)p[i];
}
template <typename T> __device__ __forceinline__ float bits_f32(uint32_t u);
template <> __device__ __forceinline__ float bits_f32<float>(uint32_t u) { return __uint_as_float(u); }
template <> __device__ __forceinline__ float bits_f32<bf16_t>(uint32_t u) { return __uint_as_float(u << 16); }

// A[d,n] = -exp(A_log[d,n]) folded with log2(e), so that exp(Delta*A) = exp2(Delta*A2)
// (mamba-rs exp_negate: out = -exp(a_log)).  Computed once per state per kernel with the
// accurate library exp.
__device__ __forceinline__ float a2_from_alog(float a_log) { return -expf(a_log) * kLog2e; }

// Raw buffer access: a per-tile buffer resource whose range ends at the end of the
// sequence (or is empty), so loads outside it return 0 and stores outside it are
// dropped by the hardware.  Lanes of padding channels use an offset >= 2^31, which is
// always outside.  This keeps every load and store of the loop unconditional.
constexpr uint32_t kBufWord3 = 0x00020000;  // gfx9-family raw buffer descriptor, word 3
constexpr uint32_t kOutside = 0x80000000u;

// lane offset + tile offset; either one outside makes the sum outside (no wrap-around)
__device__ __forceinline__ uint32_t off_add(uint32_t a, uint32_t b) {
  return ((a | b) & kOutside) ? kOutside : a + b;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t bytes) {
  const int nr = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nr, kBufWord3);
}
template <typename T> __device__ __forceinline__ float buf_ld(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ float buf_ld<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));  // bits, not a value cast
}
template <> __device__ __forceinline__ float buf_ld<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
// raw element bits (zero-extended), converted to fp32 only where the value is used, so
// that a load's wait is not pulled up to the load
template <typename T> __device__ __forceinline__ uint32_t buf_ld_raw(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ uint32_t buf_ld_raw<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <> __device__ __forceinline__ uint32_t buf_ld_raw<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
template <typename T> __device__ __forceinline__ float raw_f32(uint32_t v) {
  return std::is_same<T, float>::value ? __uint_as_float(v) : __uint_as_float(v << 16);
}
template <typename T> __device__ __forceinline__ void buf_st(float v, __amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ void buf_st<float>(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);  // bits, not a value cast
}
template <> __device__ __forceinline__ void buf_st<bf16_t>(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
}

// ---- in-row (16-lane) exchanges shared by the states-across-lanes kernels, where lane
// 16 c + n holds state n of channel c

// Halving exchanges of the in-row transpose-reduce, written as DPP adds whose bank
// masks make each instruction write only half of the row, so one register holds both
// halves' results.  One s_nop covers the DPP read-after-VALU-write wait for the whole
// block (its sources are not written inside it).
// Stage 1: partner lane i^8 (rows rotate by 8); lanes 0-7 of a row keep p[j] + partner's
// p[j], lanes 8-15 p[j+8] + partner's p[j+8] (j < 8).
__device__ __forceinline__ void row_halve_ror8(const float (&p)[16], float (&q)[8]) {
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %16, %16 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %17, %17 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %18, %18 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %19, %19 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %4, %20, %20 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %5, %21, %21 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %6, %22, %22 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %7, %23, %23 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6]), "=&v"(q[7])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]), "v"(p[8]),
        "v"(p[9]), "v"(p[10]), "v"(p[11]), "v"(p[12]), "v"(p[13]), "v"(p[14]), "v"(p[15]));
}
// Stage 2: partner = the mirror lane inside each half row (lane i^7); lanes with bit 2
// clear (banks 0 and 2) keep q[j] + partner's q[j], the others q[j+4] + partner's (j < 4).
__device__ __forceinline__ void row_halve_mirror8(const float (&q)[8], float (&r)[4]) {
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %8, %8 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %1, %9, %9 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %6, %6 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %10, %10 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %3, %7, %7 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %3, %11, %11 row_half_mirror row_mask:0xf bank_mask:0xa"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]));
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __builtin_amdgcn_update_dpp(0.f, v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppRowBcast0 = 0x150;  // row_newbcast:0 (+t: every lane of a row reads its lane t)

// sum over the 16 lanes of a row, the same value in every lane of the row (a fixed
// butterfly: quad neighbours, quads, half rows)
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<0x141>(v);  // row_half_mirror: lane i <-> 7 - i of its half row
  v += dpp_f<0x140>(v);  // row_mirror: lane i <-> 15 - i
  return v;
}
// sum over the four rows (lanes l, l ^ 16, l ^ 32, l ^ 48), the same value in each:
// permlane swaps of the halves, then of even and odd rows, ((r0 + r2) + (r1 + r3))
__device__ __forceinline__ float rows_sum4(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum over the 64 lanes of a wave, the same value in every lane, without LDS
__device__ __forceinline__ float wave_sum64(float v) { return rows_sum4(row_sum16(v)); }

// p[j] in every lane of a 16-lane row -> lane i of the row returns sum over the row of
// p[i].  Exchanges halve the values held at lane distances 8, 7, 2, 1; lane i keeps
// the half that its bit 3, 2, 1, 0 selects, so the index it ends with is i itself.
__device__ __forceinline__ float row_transpose_sum16(const float (&p)[16], int lane) {
  float q[8], r[4], s[2];
  row_halve_ror8(p, q);
  row_halve_mirror8(q, r);
  const bool b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float send = b1 ? r[j] : r[j + 2];
    const float keep = b1 ? r[j + 2] : r[j];
    s[j] = keep + dpp_f<kDppQuadXor2>(send);
  }
  const float send = b0 ? s[0] : s[1];
  const float keep = b0 ? s[1] : s[0];
  return keep + dpp_f<kDppQuadXor1>(send);
}

}  // namespace ssm
