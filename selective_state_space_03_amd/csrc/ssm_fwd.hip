// ssm_fwd.hip -- forward selective scan for gfx950.
//
// Computes, for every (batch b, channel d), the recurrence of the POPCORNBENCH
// transcript's selective_scan_kernel (state update first, readout from the updated
// state, skip term) with the discretisation and gate of mamba-rs kernels.rs
// (softplus_fwd / exp_negate / split_gate_silu, gating_backward: y = ssm_out * gate):
//   Delta = softplus(delta_raw + dt_bias), a = exp(Delta A) = exp2(Delta A2)
//   h_n  <- a h_n + (Delta x) B_n ;  y = (sum_n C_n h_n + D x) * silu(z)
//
// Work decomposition (designed for 64-lane wavefronts, not taken from the pages):
//   * one workgroup = one batch element b and a tile of 64 consecutive channels;
//     lane = channel, so every global load and store of x/delta_raw/z/y is one
//     contiguous 256 B (fp32) or 128 B (bf16) row segment per wavefront;
//   * the G wavefronts of the workgroup split the state axis: wave w owns states
//     [w*S, w*S + S) of all 64 channels and keeps them in VGPRs for the whole
//     sequence.  All 64 lanes of a wave need the same B[b,t,n] and C[b,t,n], so
//     those are wave-uniform scalar loads (SGPR operands, no VALU or LDS cost);
//   * per-(t,d) work (softplus, Delta*x, D*x, silu(z)) is done once per element
//     in a "prep" phase spread over all waves and shared through LDS, and the
//     readout sum over states is a per-wave partial in LDS that a "readout"
//     phase adds in fixed wave order -- so the result is deterministic.
// Time is walked in tiles of TT steps with one barrier per tile: between two
// barriers a wave preps tile k+1, reads out tile k-1 and scans tile k (LDS buffers
// are double / triple buffered for that).  Global loads of activations run P tiles
// ahead of the prep and the scalar loads of B/C one tile ahead of the scan, so no step
// of the scan waits on memory.  The scalar unit is shared by the four SIMDs of a CU,
// so address arithmetic is kept off it: B/C of a tile are immediate offsets from one
// base, activations a uniform row base plus a 32-bit lane offset.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

template <typename T, int S, int G, int TT, int P, bool GATED, bool MASKED>
__global__ void __launch_bounds__(64 * G)
fwd_scan_kernel(const T* __restrict__ x, const T* __restrict__ delta_raw, const T* __restrict__ z,
                const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ A_log,
                const float* __restrict__ D_skip, const float* __restrict__ dt_bias,
                const float* __restrict__ h0, T* __restrict__ y, float* __restrict__ h_final,
                int L, int Dm, int N_rt, int ngroups) {
  static_assert(P == 4, "ring slots and LDS buffer indices are derived from P == 4");
  constexpr int EPL = (TT + G - 1) / G;  // prep/readout elements per lane per tile
  // Unmasked, d_state == S*G is a compile-time constant, so every B/C load of a tile is
  // an immediate offset from one scalar base (no per-load scalar address arithmetic).
  const int N = MASKED ? N_rt : S * G;
  __shared__ float2 dd[2][TT * 64];       // (Delta, Delta*x) per (t, channel): tile k in k&1
  __shared__ float2 xz[4][TT * 64];       // (D*x, silu(z)) per (t, channel): tile k in k&3
  __shared__ float yp[2][TT * G * 64];    // per-wave partial readout per (t, wave, channel)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x / ngroups;
  const int d = (blockIdx.x % ngroups) * 64 + lane;
  const bool dvalid = d < Dm;
  const int dl = dvalid ? d : Dm - 1;  // clamped channel: loads stay in bounds
  const float bias = (dvalid && dt_bias) ? dt_bias[d] : 0.f;
  const float dsk = (dvalid && D_skip) ? D_skip[d] : 0.f;

  // this wave's states; masked states (beyond N) get A2 = 0 and B = C = 0: they stay 0
  const int n0 = wave * S;
  const int nact = N - n0 < 0 ? 0 : (N - n0 > S ? S : N - n0);  // wave-uniform
  const int64_t hb = ((int64_t)b * Dm + d) * N + n0;
  float A2[S], h[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool v = dvalid && j < nact;
    A2[j] = v ? a2_from_alog(A_log[(int64_t)d * N + n0 + j]) : 0.f;
    h[j] = (v && h0) ? h0[hb + j] : 0.f;
  }

  const int ntiles = (L + TT - 1) / TT;
  const int nfull = L / TT;              // tiles that lie entirely inside the sequence
  const int64_t row0 = (int64_t)b * L;   // row of (b, t) is row0 + t
  const int64_t tstride = (int64_t)TT * Dm;
  // per-lane element offsets inside a tile (row wave + G*i of the tile, channel dl)
  int eoff[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) eoff[i] = (wave + G * i) * Dm + dl;

  // ---- B/C: a whole tile for this wave's states in SGPRs, next tile loaded while
  // the current one is scanned
  float cb[TT][S], cc[TT][S];
  // whole tile j inside the sequence: constant offsets from one base
  auto load_bc_full = [&](int j, int t, int s) {
    const T* __restrict__ Bt = Bm + (row0 + (int64_t)j * TT) * N + n0;
    const T* __restrict__ Ct = Cm + (row0 + (int64_t)j * TT) * N + n0;
    if (MASKED) {
      cb[t][s] = s < nact ? io<T>::ld(Bt, t * N + s) : 0.f;
      cc[t][s] = s < nact ? io<T>::ld(Ct, t * N + s) : 0.f;
    } else {
      cb[t][s] = io<T>::ld(Bt, t * N + s);
      cc[t][s] = io<T>::ld(Ct, t * N + s);
    }
  };
  // partial last tile (or past the end): rows clamped, padded steps have Delta = 0
  auto load_bc_tail = [&](int j, int t, int s) {
    int r = j * TT + t;
    r = r < L ? r : L - 1;
    const int64_t o = (row0 + r) * N + n0 + (s < nact ? s : 0);
    cb[t][s] = s < nact ? io<T>::ld(Bm, o) : 0.f;
    cc[t][s] = s < nact ? io<T>::ld(Cm, o) : 0.f;
  };
  auto load_bc = [&](int j, int t, int s) {
    if (j < nfull) load_bc_full(j, t, s); else load_bc_tail(j, t, s);
  };
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int j = 0; j < S; ++j) load_bc(0, t, j);

  // ---- activations of the tiles still to prep, in a ring of P register slots: the
  // loads of tile j are issued P tiles before tile j is prepped (slot j % P)
  float px[P][EPL], pr[P][EPL], pz[P][EPL];
  auto load_tile = [&](int j, int slot) {
    if (j < nfull) {
      const int64_t base = (row0 + (int64_t)j * TT) * Dm;  // uniform
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        // with more waves than tile rows (G > TT) the extra waves have no row here
        if (wave + G * i < TT) {
          px[slot][i] = io<T>::ld(x + base, eoff[i]);
          pr[slot][i] = io<T>::ld(delta_raw + base, eoff[i]);
          pz[slot][i] = GATED ? io<T>::ld(z + base, eoff[i]) : 0.f;
        } else {
          px[slot][i] = pr[slot][i] = pz[slot][i] = 0.f;
        }
      }
    } else {  // rows past the end are clamped; prep gives them Delta = 0
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        int r = j * TT + wave + G * i;
        r = r < L ? r : L - 1;
        const int64_t base = (row0 + r) * Dm;
        px[slot][i] = io<T>::ld(x + base, dl);
        pr[slot][i] = io<T>::ld(delta_raw + base, dl);
        pz[slot][i] = GATED ? io<T>::ld(z + base, dl) : 0.f;
      }
    }
  };
  // prep of tile k: Delta and Delta*x for the scan, D*x and silu(z) for the readout.
  // Padded steps and channels get Delta = 0, which leaves the state as it is.
  auto prep = [&](int k, int slot, int dbuf, int xbuf) {
    const bool full = k < nfull;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      if (t < TT) {
        const bool v = dvalid && (full || k * TT + t < L);
        const float delta = softplus_f(pr[slot][i] + bias);
        dd[dbuf][t * 64 + lane] = v ? make_float2(delta, delta * px[slot][i]) : make_float2(0.f, 0.f);
        xz[xbuf][t * 64 + lane] = make_float2(dsk * px[slot][i], GATED ? silu_f(pz[slot][i]) : 1.f);
      }
    }
  };
  // readout of tile k: wave partials added in fixed order, plus skip, times gate
  auto readout = [&](int k, int pbuf, int xbuf) {
    const bool full = k < nfull;
    const int64_t base = (row0 + (int64_t)k * TT) * Dm;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int t = wave + G * i;
      if (t < TT && dvalid && (full || k * TT + t < L)) {
        const float2 q = xz[xbuf][t * 64 + lane];
        float s = q.x;
#pragma unroll
        for (int w = 0; w < G; ++w) s += yp[pbuf][(t * G + w) * 64 + lane];
        io<T>::st(y + base, eoff[i], s * q.y);
      }
    }
  };
  // Scan of tile k over this wave's states.  Scalar (B/C) and LDS loads share one
  // wait counter and scalar loads complete out of order, so the tile's LDS reads are
  // issued and waited for first; inside the unrolled loop the only memory operations
  // are the partial stores and the B/C loads of tile k+1.
  auto scan = [&](int k, int dbuf, int pbuf, auto&& load_next) {
    float2 v[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) v[t] = dd[dbuf][t * 64 + lane];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // s_waitcnt lgkmcnt(0)
    float* __restrict__ ypw = yp[pbuf] + wave * 64 + lane;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < S; ++j) {
        const float a = exp2_hw(v[t].x * A2[j]);
        h[j] = fmaf(a, h[j], v[t].y * cb[t][j]);
        acc = fmaf(cc[t][j], h[j], acc);
        load_next(k + 1, t, j);
      }
      ypw[t * G * 64] = acc;
    }
  };

  // prologue: tiles 0..P-1 in flight, tile 0 prepped, then tile P takes slot 0
#pragma unroll
  for (int u = 0; u < P; ++u)
    if (u < ntiles) load_tile(u, u);
  prep(0, 0, 0, 0);
  if (P < ntiles) load_tile(P, 0);
  __syncthreads();
  // main loop, unrolled by P = 4 so that ring slots and buffer indices are constants
  for (int kk = 0; kk < ntiles; kk += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int k = kk + u;
      if (k >= ntiles) break;
      if (k + 1 < ntiles) {
        prep(k + 1, (u + 1) % P, (u + 1) & 1, (u + 1) & 3);
        if (k + 1 + P < ntiles) load_tile(k + 1 + P, (u + 1) % P);
      }
      if (k >= 1) readout(k - 1, (u + 1) & 1, (u + 3) & 3);
      if (k + 1 < nfull)
        scan(k, u & 1, u & 1, load_bc_full);  // tile k+1 lies inside the sequence
      else
        scan(k, u & 1, u & 1, load_bc_tail);  // tile k+1 is partial or past the end
      __syncthreads();
    }
  }
  readout(ntiles - 1, (ntiles - 1) & 1, (ntiles - 1) & 3);

  if (h_final && dvalid) {
#pragma unroll
    for (int j = 0; j < S; ++j)
      if (j < nact) h_final[hb + j] = h[j];
  }
}

template <typename T, int S, int G, bool GATED>
hipError_t launch_cfg(const FwdArgs& a, hipStream_t stream) {
  // time tile: the B/C ring of a tile takes 2*TT*S SGPRs, so TT*S <= 16 (32 SGPRs);
  // with 16 waves the LDS partials also cap TT at 8
  constexpr int TT = G >= 16 ? 8 : (S == 1 ? 16 : (S == 2 ? 8 : 4));
  // activation prefetch depth in tiles: about 64 steps ahead of the scan
  constexpr int PF = 4;
  const int ngroups = (int)((a.dim + 63) / 64);
  const int64_t nblocks = (int64_t)ngroups * a.batch;
  if (a.dstate == S * G)
    hipLaunchKernelGGL((fwd_scan_kernel<T, S, G, TT, PF, GATED, false>), dim3((unsigned)nblocks), dim3(64 * G), 0,
                       stream, (const T*)a.x, (const T*)a.delta_raw, (const T*)a.z, (const T*)a.B,
                       (const T*)a.C, a.A_log, a.D_skip, a.dt_bias, a.h0, (T*)a.y, a.h_final, (int)a.seqlen,
                       (int)a.dim, a.dstate, ngroups);
  else
    hipLaunchKernelGGL((fwd_scan_kernel<T, S, G, TT, PF, GATED, true>), dim3((unsigned)nblocks), dim3(64 * G), 0,
                       stream, (const T*)a.x, (const T*)a.delta_raw, (const T*)a.z, (const T*)a.B,
                       (const T*)a.C, a.A_log, a.D_skip, a.dt_bias, a.h0, (T*)a.y, a.h_final, (int)a.seqlen,
                       (int)a.dim, a.dstate, ngroups);
  return hipGetLastError();
}

// States per wave S: fewer states per wave means more wavefronts (more parallelism
// and latency hiding) but more LDS traffic per state update.  Default: one state per
// wave (measured fastest on MI355X for d_state = 16; SSM_FWD_STATES_PER_WAVE overrides).
int pick_states_per_wave(const FwdArgs& a, int ns) {
  if (const char* e = getenv("SSM_FWD_STATES_PER_WAVE")) {
    const int v = atoi(e);
    if (v == 1 || v == 2 || v == 4 || v == ns) return v;
  }
  return 1;
}

template <typename T, bool GATED>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int ns = a.dstate <= 4 ? 4 : (a.dstate <= 8 ? 8 : 16);
  const int s = pick_states_per_wave(a, ns);
  if (ns == 16) {
    switch (s) {
      case 2: return launch_cfg<T, 2, 8, GATED>(a, stream);
      case 4: return launch_cfg<T, 4, 4, GATED>(a, stream);
      case 16: return launch_cfg<T, 16, 1, GATED>(a, stream);
      default: return launch_cfg<T, 1, 16, GATED>(a, stream);
    }
  }
  if (ns == 8) {
    switch (s) {
      case 2: return launch_cfg<T, 2, 4, GATED>(a, stream);
      case 8: return launch_cfg<T, 8, 1, GATED>(a, stream);
      default: return launch_cfg<T, 1, 8, GATED>(a, stream);
    }
  }
  switch (s) {
    case 4: return launch_cfg<T, 4, 1, GATED>(a, stream);
    default: return launch_cfg<T, 1, 4, GATED>(a, stream);
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.bf16) return a.z ? launch_t<bf16_t, true>(a, stream) : launch_t<bf16_t, false>(a, stream);
  return a.z ? launch_t<float, true>(a, stream) : launch_t<float, false>(a, stream);
}

}  // namespace ssm
