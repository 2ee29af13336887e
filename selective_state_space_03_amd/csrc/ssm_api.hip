// ssm_api.hip -- the extern "C" entry points declared in include/ssm_scan.h and
// include/ssm_conv1d.h.
// Every argument is validated before anything is enqueued; launch errors are mapped
// to SSM_ERR_HIP.  No exception crosses the boundary.
#include <stdint.h>

#include <new>

#include "../../include/ssm_conv1d.h"
#include "../../include/ssm_decode.h"
#include "../../include/ssm_scan.h"
#include "ssm_internal.h"

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool dims_ok(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  if (batch < 1 || seqlen < 1 || d_inner < 1 || d_state < 1 || d_state > 16) return false;
  // element counts must fit comfortably in int64 byte offsets and grid sizes
  const int64_t lim = (int64_t)1 << 40;
  if (batch > lim / seqlen) return false;
  if (batch * seqlen > lim / d_inner) return false;
  if ((d_inner + 63) / 64 * batch > ((int64_t)1 << 31) - 1) return false;
  return true;
}

size_t esize(int io_dtype) { return io_dtype == SSM_BF16 ? 2 : 4; }

bool conv_dims_ok(int64_t batch, int64_t seqlen, int64_t dim, int64_t width) {
  if (batch < 1 || seqlen < 1 || dim < 1 || width < 1 || width > 8) return false;
  const int64_t lim = (int64_t)1 << 40;
  if (batch > lim / seqlen) return false;
  if (batch * seqlen > lim / dim) return false;
  // grids are 1-D: channel groups x time groups x batch (and batch * dim for a step)
  if ((dim + 63) / 64 * ((seqlen + 63) / 64) * batch > ((int64_t)1 << 31) - 1) return false;
  return true;
}

// Options of the _ex entry points: clamp bounds (dt_max <= 0: no upper bound) and the
// backward-only state gradients.  NULL options are the defaults.
bool options_ok(const ssm_scan_options* o, bool backward, float* lo, float* hi, bool step = false) {
  *lo = 0.f;
  *hi = __builtin_inff();
  if (!o) return true;
  if (!(o->dt_min >= 0.f) || o->dt_max != o->dt_max) return false;  // negative or NaN
  if (o->dt_max > 0.f) {
    if (o->dt_min > o->dt_max) return false;
    *hi = o->dt_max;
  }
  *lo = o->dt_min;
  if (!backward && (o->dh_final || o->dh0)) return false;
  if (step && o->chunk_states) return false;
  return true;
}

int64_t state_chunks(int64_t seqlen) { return (seqlen + ssm::kStateChunk - 1) / ssm::kStateChunk; }
// one batch element's chunk states are addressed with 31-bit offsets
bool chunk_states_fit(int64_t seqlen, int64_t d_inner, int64_t d_state) {
  return (uint64_t)state_chunks(seqlen) * (uint64_t)d_state * (uint64_t)d_inner * 4 < ((uint64_t)1 << 31);
}

// The conv1d backward with a caller workspace, or (use_scratch) with the library's
// fixed per-device scratch, which must hold the workspace the sizes need.  Every check
// runs before the scratch address is looked up or anything is launched.
int conv1d_bwd_common(const void* x, const float* weight, const float* bias, const void* dout, void* dx,
                      float* dweight, float* dbias, void* workspace, size_t workspace_bytes, bool use_scratch,
                      int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int activation, int io_dtype,
                      hipStream_t stream) {
  if (!x || !weight || !dout || !dx) return SSM_ERR_NULL;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (activation != SSM_ACT_NONE && activation != SSM_ACT_SILU) return SSM_ERR_UNSUPPORTED;
  if (!conv_dims_ok(batch, seqlen, dim, width)) return SSM_ERR_DIM;
  if (io_dtype != SSM_F32) return SSM_ERR_UNSUPPORTED;
  const ssm::ConvBwdLayout l = ssm::conv_bwd_layout(batch, seqlen, dim, width);
  if (use_scratch) {
    if (l.total > ssm::kConvScratchBytes) return SSM_ERR_SCRATCH;
  } else {
    if (!workspace) return SSM_ERR_WORKSPACE;
    if (workspace_bytes < l.total || !aligned(workspace, 256)) return SSM_ERR_WORKSPACE;
  }
  const void* all[] = {x, weight, bias, dout, dx, dweight, dbias};
  for (const void* p : all)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  const size_t E = (size_t)batch * seqlen * dim, W = (size_t)dim * width;
  const Range ins[] = {rng(x, E * 4), rng(weight, W * 4), rng(bias, bias ? dim * 4 : 0), rng(dout, E * 4)};
  const Range outs[] = {rng(dx, E * 4), rng(dweight, dweight ? W * 4 : 0), rng(dbias, dbias ? dim * 4 : 0),
                        rng(workspace, use_scratch ? 0 : l.total)};
  const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
  for (int i = 0; i < nout; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }
  if (use_scratch && ssm::conv_scratch(&workspace) != hipSuccess) return SSM_ERR_HIP;
  ssm::ConvArgs a{};
  a.x = x; a.w = weight; a.bias = bias; a.dout = dout; a.dx = dx; a.dw = dweight; a.dbias = dbias;
  a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.width = (int)width;
  a.silu = activation == SSM_ACT_SILU; a.bf16 = false;
  return ssm::launch_conv_bwd(a, workspace, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_NULL: return "SSM_ERR_NULL: a required pointer is NULL";
    case SSM_ERR_DIM: return "SSM_ERR_DIM: a size is out of range";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: request not handled by this library";
    case SSM_ERR_ALIGN: return "SSM_ERR_ALIGN: a pointer is not aligned to its element size";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing or too small";
    case SSM_ERR_ALIAS: return "SSM_ERR_ALIAS: an output overlaps an input";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: the HIP runtime reported an error";
    case SSM_ERR_ARG: return "SSM_ERR_ARG: an option value is out of range";
    case SSM_ERR_SCRATCH: return "SSM_ERR_SCRATCH: the sizes need more than the library's fixed scratch";
    default: return "unknown ssm_status";
  }
}

size_t ssm_scan_chunk_states_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  if (!dims_ok(batch, seqlen, d_inner, d_state)) return 0;
  return (size_t)batch * state_chunks(seqlen) * d_state * d_inner * 4;
}

size_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                    int io_dtype) {
  (void)io_dtype;
  if (!dims_ok(batch, seqlen, d_inner, d_state)) return 0;
  const ssm::FwdSplit sp = ssm::fwd_split(batch, seqlen, d_inner, (int)d_state);
  return sp.nseg > 1 ? sp.total : 0;
}

int ssm_scan_fwd(const void* x, const void* delta_raw, const void* z, const void* B, const void* C,
                 const float* A_log, const float* D_skip, const float* dt_bias, const float* h0, void* y,
                 float* h_final, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                 int io_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ssm_scan_fwd_ex(x, delta_raw, z, B, C, A_log, D_skip, dt_bias, h0, y, h_final, batch, seqlen,
                         d_inner, d_state, io_dtype, workspace, workspace_bytes, nullptr, stream);
}

int ssm_scan_fwd_ex(const void* x, const void* delta_raw, const void* z, const void* B, const void* C,
                    const float* A_log, const float* D_skip, const float* dt_bias, const float* h0, void* y,
                    float* h_final, int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                    int io_dtype, void* workspace, size_t workspace_bytes, const ssm_scan_options* options,
                    hipStream_t stream) {
  if (!x || !delta_raw || !B || !C || !A_log || !y) return SSM_ERR_NULL;
  float dt_lo, dt_hi;
  if (!options_ok(options, false, &dt_lo, &dt_hi)) return SSM_ERR_ARG;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (!dims_ok(batch, seqlen, d_inner, d_state)) return SSM_ERR_DIM;
  // per-tile buffer offsets of the forward kernel are 32-bit: a 16-row tile of one
  // batch element must stay below 2^31 bytes
  if (d_inner > ((int64_t)1 << 24) || seqlen > ((int64_t)1 << 30)) return SSM_ERR_DIM;
  const size_t es = esize(io_dtype);
  // the forward addresses one batch element's [seqlen, d_inner] and [seqlen, d_state]
  // slices with 31-bit offsets
  if ((uint64_t)seqlen * (uint64_t)(d_inner > d_state ? d_inner : d_state) * es >= ((uint64_t)1 << 31))
    return SSM_ERR_UNSUPPORTED;
  const void* io_in[] = {x, delta_raw, z, B, C};
  for (const void* p : io_in)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  float* chunk_states = options ? options->chunk_states : nullptr;
  // saved chunk states come from the states-across-lanes kernel (d_state 9..16)
  if (chunk_states && (d_state < 9 || !chunk_states_fit(seqlen, d_inner, d_state))) return SSM_ERR_UNSUPPORTED;
  const void* f_in[] = {A_log, D_skip, dt_bias, h0, h_final, chunk_states};
  for (const void* p : f_in)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  if (!aligned(y, es)) return SSM_ERR_ALIGN;
  // the time-split path (long sequences of few channels) needs the workspace; whether
  // it is taken depends on the sizes alone
  const ssm::FwdSplit sp = ssm::fwd_split(batch, seqlen, d_inner, (int)d_state);
  const size_t ws_used = sp.nseg > 1 ? sp.total : 0;
  if (ws_used && (!workspace || workspace_bytes < ws_used || !aligned(workspace, 256))) return SSM_ERR_WORKSPACE;
  const size_t E = (size_t)batch * seqlen * d_inner, S = (size_t)batch * seqlen * d_state;
  const size_t H = (size_t)batch * d_inner * d_state;
  const Range ins[] = {rng(x, E * es), rng(delta_raw, E * es), rng(z, z ? E * es : 0), rng(B, S * es),
                       rng(C, S * es), rng(A_log, (size_t)d_inner * d_state * 4),
                       rng(D_skip, D_skip ? d_inner * 4 : 0), rng(dt_bias, dt_bias ? d_inner * 4 : 0),
                       rng(h0, h0 ? H * 4 : 0)};
  const Range outs[] = {rng(y, E * es), rng(h_final, h_final ? H * 4 : 0),
                        rng(chunk_states, chunk_states ? ssm_scan_chunk_states_bytes(batch, seqlen, d_inner, d_state) : 0),
                        rng(workspace, ws_used)};
  const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
  for (int i = 0; i < nout; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }

  ssm::FwdArgs a;
  a.x = x; a.delta_raw = delta_raw; a.z = z; a.B = B; a.C = C; a.A_log = A_log; a.D_skip = D_skip;
  a.dt_bias = dt_bias; a.h0 = h0; a.y = y; a.h_final = h_final;
  a.batch = batch; a.seqlen = seqlen; a.dim = d_inner; a.dstate = (int)d_state;
  a.bf16 = io_dtype == SSM_BF16;
  a.dt_lo = dt_lo; a.dt_hi = dt_hi; a.chunk_states = chunk_states;
  a.workspace = ws_used ? workspace : nullptr;
  return ssm::launch_fwd(a, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_step(float* state, const void* x, const void* delta_raw, const void* z, const void* B,
                  const void* C, const float* A_log, const float* D_skip, const float* dt_bias, void* y,
                  int64_t batch, int64_t d_inner, int64_t d_state, int io_dtype, hipStream_t stream) {
  return ssm_scan_step_ex(state, x, delta_raw, z, B, C, A_log, D_skip, dt_bias, y, batch, d_inner, d_state,
                          io_dtype, nullptr, stream);
}

int ssm_scan_step_ex(float* state, const void* x, const void* delta_raw, const void* z, const void* B,
                     const void* C, const float* A_log, const float* D_skip, const float* dt_bias, void* y,
                     int64_t batch, int64_t d_inner, int64_t d_state, int io_dtype,
                     const ssm_scan_options* options, hipStream_t stream) {
  if (!state || !x || !delta_raw || !B || !C || !A_log || !y) return SSM_ERR_NULL;
  float dt_lo, dt_hi;
  if (!options_ok(options, false, &dt_lo, &dt_hi, true)) return SSM_ERR_ARG;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (!dims_ok(batch, 1, d_inner, d_state)) return SSM_ERR_DIM;
  if (batch * d_inner * 4 >= ((int64_t)1 << 31) * 256) return SSM_ERR_DIM;  // grid limit
  const size_t es = esize(io_dtype);
  const void* io_in[] = {x, delta_raw, z, B, C, y};
  for (const void* p : io_in)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* f_in[] = {state, A_log, D_skip, dt_bias};
  for (const void* p : f_in)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  const size_t E = (size_t)batch * d_inner, S = (size_t)batch * d_state, H = E * d_state;
  const Range ins[] = {rng(x, E * es), rng(delta_raw, E * es), rng(z, z ? E * es : 0), rng(B, S * es),
                       rng(C, S * es), rng(A_log, (size_t)d_inner * d_state * 4),
                       rng(D_skip, D_skip ? d_inner * 4 : 0), rng(dt_bias, dt_bias ? d_inner * 4 : 0)};
  const Range outs[] = {rng(state, H * 4), rng(y, E * es)};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return SSM_ERR_ALIAS;
  if (overlap(outs[0], outs[1])) return SSM_ERR_ALIAS;

  ssm::StepArgs a;
  a.state = state; a.x = x; a.delta_raw = delta_raw; a.z = z; a.B = B; a.C = C; a.A_log = A_log;
  a.D_skip = D_skip; a.dt_bias = dt_bias; a.y = y;
  a.batch = batch; a.dim = d_inner; a.dstate = (int)d_state; a.bf16 = io_dtype == SSM_BF16;
  a.dt_lo = dt_lo; a.dt_hi = dt_hi;
  return ssm::launch_step(a, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_decode_step(void* conv_state, const void* x, const float* conv_weight, const float* conv_bias,
                    int64_t width, int activation, float* state, const void* delta_raw, const void* z,
                    const void* B, const void* C, const float* A_log, const float* D_skip,
                    const float* dt_bias, void* u, void* y, int64_t batch, int64_t d_inner, int64_t d_state,
                    int io_dtype, const ssm_scan_options* options, hipStream_t stream) {
  if (!state || !x || !conv_weight || !delta_raw || !B || !C || !A_log || !y || (width > 1 && !conv_state))
    return SSM_ERR_NULL;
  float dt_lo, dt_hi;
  if (!options_ok(options, false, &dt_lo, &dt_hi, true)) return SSM_ERR_ARG;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (activation != SSM_ACT_NONE && activation != SSM_ACT_SILU) return SSM_ERR_UNSUPPORTED;
  if (!dims_ok(batch, 1, d_inner, d_state) || !conv_dims_ok(batch, 1, d_inner, width)) return SSM_ERR_DIM;
  if (batch * d_inner * 4 >= ((int64_t)1 << 31) * 256) return SSM_ERR_DIM;  // grid limit
  const size_t es = esize(io_dtype);
  const void* io_ptrs[] = {x, delta_raw, z, B, C, y, u, conv_state};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* f_ptrs[] = {state, A_log, D_skip, dt_bias, conv_weight, conv_bias};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  const size_t E = (size_t)batch * d_inner, S = (size_t)batch * d_state, H = E * d_state;
  const Range ins[] = {rng(x, E * es), rng(delta_raw, E * es), rng(z, z ? E * es : 0), rng(B, S * es),
                       rng(C, S * es), rng(A_log, (size_t)d_inner * d_state * 4),
                       rng(D_skip, D_skip ? d_inner * 4 : 0), rng(dt_bias, dt_bias ? d_inner * 4 : 0),
                       rng(conv_weight, (size_t)d_inner * width * 4), rng(conv_bias, conv_bias ? d_inner * 4 : 0)};
  const Range outs[] = {rng(state, H * 4), rng(y, E * es), rng(u, u ? E * es : 0),
                        rng(conv_state, width > 1 ? E * (width - 1) * es : 0)};
  const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
  for (int i = 0; i < nout; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }

  ssm::StepArgs a;
  a.state = state; a.x = x; a.delta_raw = delta_raw; a.z = z; a.B = B; a.C = C; a.A_log = A_log;
  a.D_skip = D_skip; a.dt_bias = dt_bias; a.y = y;
  a.batch = batch; a.dim = d_inner; a.dstate = (int)d_state; a.bf16 = io_dtype == SSM_BF16;
  a.dt_lo = dt_lo; a.dt_hi = dt_hi;
  a.conv_state = width > 1 ? conv_state : nullptr; a.conv_w = conv_weight; a.conv_b = conv_bias; a.u = u;
  a.width = (int)width; a.silu = activation == SSM_ACT_SILU;
  return ssm::launch_step(a, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                                    int io_dtype) {
  (void)io_dtype;
  if (!dims_ok(batch, seqlen, d_inner, d_state)) return 0;
  return ssm::bwd_layout(batch, seqlen, d_inner, (int)d_state).total;
}

int ssm_scan_bwd(const void* x, const void* delta_raw, const void* z, const void* B, const void* C,
                 const float* A_log, const float* D_skip, const float* dt_bias, const float* h0,
                 const void* dy, void* dx, void* ddelta_raw, void* dz, float* dB, float* dC, float* dA_log,
                 float* dD, float* d_dt_bias, void* workspace, size_t workspace_bytes, int64_t batch,
                 int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype, hipStream_t stream) {
  return ssm_scan_bwd_ex(x, delta_raw, z, B, C, A_log, D_skip, dt_bias, h0, dy, dx, ddelta_raw, dz, dB, dC,
                         dA_log, dD, d_dt_bias, workspace, workspace_bytes, batch, seqlen, d_inner, d_state,
                         io_dtype, nullptr, stream);
}

int ssm_scan_bwd_ex(const void* x, const void* delta_raw, const void* z, const void* B, const void* C,
                    const float* A_log, const float* D_skip, const float* dt_bias, const float* h0,
                    const void* dy, void* dx, void* ddelta_raw, void* dz, float* dB, float* dC, float* dA_log,
                    float* dD, float* d_dt_bias, void* workspace, size_t workspace_bytes, int64_t batch,
                    int64_t seqlen, int64_t d_inner, int64_t d_state, int io_dtype,
                    const ssm_scan_options* options, hipStream_t stream) {
  if (!x || !delta_raw || !B || !C || !A_log || !dy || !dx || !ddelta_raw || !dB || !dC) return SSM_ERR_NULL;
  if (z && !dz) return SSM_ERR_NULL;
  float dt_lo, dt_hi;
  if (!options_ok(options, true, &dt_lo, &dt_hi)) return SSM_ERR_ARG;
  const float* dh_final = options ? options->dh_final : nullptr;
  float* dh0 = options ? options->dh0 : nullptr;
  const float* chunk_states = options ? options->chunk_states : nullptr;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (!dims_ok(batch, seqlen, d_inner, d_state)) return SSM_ERR_DIM;
  // the backward addresses one batch element's [seqlen, d_inner] slice and its chunk
  // states with 31-bit offsets
  if ((uint64_t)seqlen * (uint64_t)(d_inner > d_state ? d_inner : d_state) * esize(io_dtype) >= ((uint64_t)1 << 31) ||
      !chunk_states_fit(seqlen, d_inner, d_state))
    return SSM_ERR_UNSUPPORTED;
  if (!workspace) return SSM_ERR_WORKSPACE;
  const ssm::BwdLayout l = ssm::bwd_layout(batch, seqlen, d_inner, (int)d_state);
  if (workspace_bytes < l.total || !aligned(workspace, 256)) return SSM_ERR_WORKSPACE;
  const size_t es = esize(io_dtype);
  const void* io_ptrs[] = {x, delta_raw, z, B, C, dy, dx, ddelta_raw, dz};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  if (chunk_states && !chunk_states_fit(seqlen, d_inner, d_state)) return SSM_ERR_UNSUPPORTED;
  const void* f32_ptrs[] = {A_log, D_skip, dt_bias, h0, dB, dC, dA_log, dD, d_dt_bias, dh_final, dh0, chunk_states};
  for (const void* p : f32_ptrs)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  const size_t E = (size_t)batch * seqlen * d_inner, S = (size_t)batch * seqlen * d_state;
  const size_t H = (size_t)batch * d_inner * d_state, P = (size_t)d_inner * d_state;
  const Range ins[] = {rng(x, E * es), rng(delta_raw, E * es), rng(z, z ? E * es : 0), rng(B, S * es),
                       rng(C, S * es), rng(A_log, P * 4), rng(D_skip, D_skip ? d_inner * 4 : 0),
                       rng(dt_bias, dt_bias ? d_inner * 4 : 0), rng(h0, h0 ? H * 4 : 0), rng(dy, E * es),
                       rng(dh_final, dh_final ? H * 4 : 0),
                       rng(chunk_states, chunk_states ? ssm_scan_chunk_states_bytes(batch, seqlen, d_inner, d_state) : 0)};
  const Range outs[] = {rng(dx, E * es), rng(ddelta_raw, E * es), rng(dz, dz && z ? E * es : 0),
                        rng(dB, S * 4), rng(dC, S * 4), rng(dA_log, dA_log ? P * 4 : 0),
                        rng(dD, dD ? d_inner * 4 : 0), rng(d_dt_bias, d_dt_bias ? d_inner * 4 : 0),
                        rng(workspace, l.total), rng(dh0, dh0 ? H * 4 : 0)};
  const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
  for (int i = 0; i < nout; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return SSM_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return SSM_ERR_ALIAS;
  }

  ssm::BwdArgs a;
  a.x = x; a.delta_raw = delta_raw; a.z = z; a.B = B; a.C = C; a.A_log = A_log; a.D_skip = D_skip;
  a.dt_bias = dt_bias; a.h0 = h0; a.dy = dy; a.dx = dx; a.ddelta_raw = ddelta_raw;
  a.dz = z ? dz : nullptr; a.bf16 = io_dtype == SSM_BF16; a.dB = dB; a.dC = dC; a.dA_log = dA_log; a.dD = dD;
  a.d_dt_bias = d_dt_bias; a.batch = batch; a.seqlen = seqlen; a.dim = d_inner; a.dstate = (int)d_state;
  a.dh_final = dh_final; a.dh0 = dh0; a.dt_lo = dt_lo; a.dt_hi = dt_hi; a.chunk_states = chunk_states;
  return ssm::launch_bwd(a, workspace, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

// ---------------------------------------------------------------- conv1d

int ssm_conv1d_fwd(const void* x, const float* weight, const float* bias, void* out, int64_t batch,
                   int64_t seqlen, int64_t dim, int64_t width, int activation, int io_dtype,
                   hipStream_t stream) {
  if (!x || !weight || !out) return SSM_ERR_NULL;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (activation != SSM_ACT_NONE && activation != SSM_ACT_SILU) return SSM_ERR_UNSUPPORTED;
  if (!conv_dims_ok(batch, seqlen, dim, width)) return SSM_ERR_DIM;
  const size_t es = esize(io_dtype);
  if (!aligned(x, es) || !aligned(out, es) || !aligned(weight, 4) || (bias && !aligned(bias, 4)))
    return SSM_ERR_ALIGN;
  const size_t E = (size_t)batch * seqlen * dim;
  const Range o = rng(out, E * es);
  if (overlap(o, rng(x, E * es)) || overlap(o, rng(weight, (size_t)dim * width * 4)) ||
      overlap(o, rng(bias, bias ? dim * 4 : 0)))
    return SSM_ERR_ALIAS;
  ssm::ConvArgs a{};
  a.x = x; a.w = weight; a.bias = bias; a.out = out;
  a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.width = (int)width;
  a.silu = activation == SSM_ACT_SILU; a.bf16 = io_dtype == SSM_BF16;
  return ssm::launch_conv_fwd(a, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_conv1d_step(void* conv_state, const void* x, const float* weight, const float* bias, void* out,
                    int64_t batch, int64_t dim, int64_t width, int activation, int io_dtype,
                    hipStream_t stream) {
  if (!x || !weight || !out || (width > 1 && !conv_state)) return SSM_ERR_NULL;
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (activation != SSM_ACT_NONE && activation != SSM_ACT_SILU) return SSM_ERR_UNSUPPORTED;
  if (!conv_dims_ok(batch, 1, dim, width)) return SSM_ERR_DIM;
  if (batch * dim > ((int64_t)1 << 31) * 255) return SSM_ERR_DIM;  // grid limit
  const size_t es = esize(io_dtype);
  if (!aligned(x, es) || !aligned(out, es) || !aligned(conv_state, es) || !aligned(weight, 4) ||
      (bias && !aligned(bias, 4)))
    return SSM_ERR_ALIGN;
  const size_t E = (size_t)batch * dim;
  const Range ins[] = {rng(x, E * es), rng(weight, (size_t)dim * width * 4), rng(bias, bias ? dim * 4 : 0)};
  const Range outs[] = {rng(out, E * es), rng(conv_state, width > 1 ? E * (width - 1) * es : 0)};
  for (const Range& r : outs)
    for (const Range& i : ins)
      if (overlap(r, i)) return SSM_ERR_ALIAS;
  if (overlap(outs[0], outs[1])) return SSM_ERR_ALIAS;
  ssm::ConvArgs a{};
  a.x = x; a.w = weight; a.bias = bias; a.out = out; a.state = conv_state;
  a.batch = batch; a.seqlen = 1; a.dim = dim; a.width = (int)width;
  a.silu = activation == SSM_ACT_SILU; a.bf16 = io_dtype == SSM_BF16;
  return ssm::launch_conv_step(a, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

size_t ssm_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int io_dtype) {
  (void)io_dtype;
  if (!conv_dims_ok(batch, seqlen, dim, width)) return 0;
  return ssm::conv_bwd_layout(batch, seqlen, dim, width).total;
}

int ssm_conv1d_bwd(const void* x, const float* weight, const float* bias, const void* dout, void* dx,
                   float* dweight, float* dbias, void* workspace, size_t workspace_bytes, int64_t batch,
                   int64_t seqlen, int64_t dim, int64_t width, int activation, int io_dtype,
                   hipStream_t stream) {
  return conv1d_bwd_common(x, weight, bias, dout, dx, dweight, dbias, workspace, workspace_bytes, false, batch,
                           seqlen, dim, width, activation, io_dtype, stream);
}

int ssm_conv1d_bwd_noalloc(const void* x, const float* weight, const float* bias, const void* dout, void* dx,
                           float* dweight, float* dbias, int64_t batch, int64_t seqlen, int64_t dim,
                           int64_t width, int activation, int io_dtype, hipStream_t stream) {
  return conv1d_bwd_common(x, weight, bias, dout, dx, dweight, dbias, nullptr, 0, true, batch, seqlen, dim, width,
                           activation, io_dtype, stream);
}

}  // extern "C"
