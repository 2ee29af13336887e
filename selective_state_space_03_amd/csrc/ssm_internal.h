// ssm_internal.h -- launch interface between the C ABI (ssm_api.hip) and the kernels.
// Host-side only declarations; arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

struct FwdArgs {
  const void* x;
  const void* delta_raw;
  const void* z;  // nullable
  const void* B;
  const void* C;
  const float* A_log;
  const float* D_skip;   // nullable
  const float* dt_bias;  // nullable
  const float* h0;       // nullable
  void* y;
  float* h_final;  // nullable
  int64_t batch, seqlen, dim;
  int dstate;
  int bf16;  // io dtype is bf16
  float dt_lo = 0.f, dt_hi = __builtin_inff();  // clamp of Delta (none by default)
  float* chunk_states = nullptr;  // [B, ceil(L/16), N, D]: state entering each 16-step chunk
  void* workspace = nullptr;      // the time-split path's workspace (FwdSplit::total bytes)
};
constexpr int kStateChunk = 16;  // steps per saved chunk state (forward tile = backward chunk)

// Time split of the forward: sequences too long for the channels alone to fill the chip
// are cut into nseg segments of seglen steps (a multiple of 16).  nseg == 1: unsplit,
// no workspace.  Workspace: the state entering each segment [B, nseg, N, D] fp32 (first
// the local end states), then the segments' step sums [B, nseg, D] fp32.
struct FwdSplit {
  int64_t nseg, seglen;
  size_t off_sumd, total;
};
FwdSplit fwd_split(int64_t batch, int64_t seqlen, int64_t dim, int dstate);

struct StepArgs {
  float* state;
  const void* x;  // with a conv1d step first: the token before the convolution
  const void* delta_raw;
  const void* z;  // nullable
  const void* B;
  const void* C;
  const float* A_log;
  const float* D_skip;   // nullable
  const float* dt_bias;  // nullable
  void* y;
  int64_t batch, dim;
  int dstate;
  int bf16;
  float dt_lo = 0.f, dt_hi = __builtin_inff();  // clamp of Delta (none by default)
  // decode: the token first goes through the depthwise conv1d step (width > 0):
  // conv_state [B, D, width - 1] io dtype, read and shifted in place; conv_w [D, width];
  // conv_b [D] nullable; u [B, D] io dtype, nullable (the convolution's output)
  void* conv_state = nullptr;
  const float* conv_w = nullptr;
  const float* conv_b = nullptr;
  void* u = nullptr;
  int width = 0;
  bool silu = false;
};

struct BwdArgs {
  const void* x;  // x, delta_raw, z, B, C, dy, dx, ddelta_raw, dz: io dtype
  const void* delta_raw;
  const void* z;  // nullable
  const void* B;
  const void* C;
  const float* A_log;
  const float* D_skip;   // nullable
  const float* dt_bias;  // nullable
  const float* h0;       // nullable
  const void* dy;
  void* dx;
  void* ddelta_raw;
  void* dz;  // non-null iff z
  float* dB;
  float* dC;
  float* dA_log;     // nullable
  float* dD;         // nullable
  float* d_dt_bias;  // nullable
  const float* dh_final = nullptr;  // [B, D, N]: gradient reaching h_final (nullable: zero)
  float* dh0 = nullptr;             // [B, D, N]: gradient of h0 (nullable: not written)
  const float* chunk_states = nullptr;  // the forward's saved chunk states (nullable: recomputed)
  int64_t batch, seqlen, dim;
  int dstate;
  int bf16;  // io dtype is bf16
  float dt_lo = 0.f, dt_hi = __builtin_inff();  // clamp of Delta (none by default)
};

// Workspace layout of the backward (byte offsets into one caller buffer).  Two paths,
// chosen by the sizes: "fused" (each wavefront walks its channels' whole sequence; the
// chunk states come from the forward or from a states-only forward pass into off_cs)
// when batch x ceil(dim / 4) >= 1024 or seqlen < 1024, else "segments" (time cut into
// segments processed in parallel, as the time-split forward does).
struct BwdLayout {
  bool fused;
  size_t off_cs;     // fused: chunk states [B, nchunks, N, D] when the forward did not save them
  int chunk;         // time steps per chunk (the recompute window)
  int64_t nchunks;   // ceil(seqlen / chunk)
  int64_t ngroups;   // ceil(dim / 64) channel groups
  int64_t segc;      // chunks per segment (segments are processed in parallel)
  int64_t nseg;      // ceil(nchunks / segc)
  size_t off_hrel, off_cumd, off_hseg, off_sdseg, off_gseg, off_hin, off_gin, off_dbc, off_dparam, total;
};
BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int dstate);

// depthwise causal conv1d (+ SiLU)
struct ConvArgs {
  const void* x;       // [B, L, D] io dtype (a step: [B, D])
  const float* w;      // [D, K]
  const float* bias;   // [D], nullable
  void* out;           // like x
  void* state;         // step only: [B, D, K-1] io dtype, read and written
  const void* dout;    // backward only, fp32
  void* dx;            // backward only, fp32
  float* dw;           // backward only, [D, K], nullable
  float* dbias;        // backward only, [D], nullable
  int64_t batch, seqlen, dim;
  int width;
  bool silu, bf16;
};
struct ConvBwdLayout {
  int64_t ntg;         // time groups (one tile per wave) per batch element
  int64_t tgs;         // time groups per segment (one workgroup)
  int64_t nseg;        // segments per batch element
  size_t off_dw, off_db, total;
};
ConvBwdLayout conv_bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t width);
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t stream);
hipError_t launch_conv_step(const ConvArgs& a, hipStream_t stream);
hipError_t launch_conv_bwd(const ConvArgs& a, void* workspace, hipStream_t stream);
// the no-allocation backward's fixed scratch: its size, and its device address on the
// current device (resolved once per device)
constexpr size_t kConvScratchBytes = (size_t)16 << 20;
hipError_t conv_scratch(void** out);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// the states-only forward: writes a.chunk_states and nothing else (y, h_final unused)
hipError_t launch_fwd_states(const FwdArgs& a, hipStream_t stream);
// the fused backward (ssm_bwd_fused.hip): per-workgroup dB/dC partials
// [B, bwd_fused_groups(D), L, N], dA partials [B, N, D], dD and d_dt_bias partials [B, D]
int64_t bwd_fused_groups(int64_t dim);
hipError_t launch_bwd_fused(const BwdArgs& a, const float* chunk_states, float* pdB, float* pdC, float* pdA,
                            float* pdD, float* pdb, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, void* workspace, hipStream_t stream);

}  // namespace ssm
