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

}  // namespace ssm
