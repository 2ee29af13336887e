"""fp64 oracle of the Mamba-2 SSD scan, forward and backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library.

What is computed.  The SSD layer of Mamba-2, whose chunked kernels the
pretraining_mamba2_outer page deterministic_backward.py drives (its module list:
ssd_combined, ssd_chunk_state, ssd_state_passing, ssd_chunk_scan, ssd_bmm), is the
selective recurrence with one scalar decay rate A per head: the cumsum arguments of
ordered_cumsum give A one value per head and dt one value per (batch, step, head).
Per (batch b, head h) the state is a [headdim P, d_state N] matrix:
    state_t = exp(dt_t * A[h]) * state_{t-1} + dt_t * outer(x_t, B_t)
    y_t     = state_t @ C_t + D[h] * x_t
with dt_t = dt_out[b, t, h] (the discretised, clamped step of the chunk cumsum),
x_t = x[b, t, h, :], and B_t, C_t = B[b, t, :], C[b, t, :] shared by every head (one
B/C group).  The readout uses the updated state, as in the Mamba selective scan.
This is the plain definition, walked sequentially in t; the chunked form that the
GPU computes reaches the same values up to rounding.  The backward is the reverse
(adjoint) recurrence of the same definition, pinned by central differences.
"""
from __future__ import annotations

import numpy as np


def ssd_scan_fwd(x, dt_out, A, B, C, D=None, h0=None):
    """x [batch, seqlen, heads, P], dt_out [batch, seqlen, heads], A [heads],
    B, C [batch, seqlen, N], D [heads] or None, h0 [batch, heads, P, N] or None
    -> {"y" [batch, seqlen, heads, P], "h_final" [batch, heads, P, N]}"""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt_out, np.float64)
    A = np.asarray(A, np.float64)
    Bm = np.asarray(B, np.float64)
    Cm = np.asarray(C, np.float64)
    b, L, H, P = x.shape
    N = Bm.shape[-1]
    Dv = np.zeros(H) if D is None else np.asarray(D, np.float64)
    y = np.zeros((b, L, H, P))
    hf = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            s = np.zeros((P, N)) if h0 is None else np.array(h0[bi, h], np.float64)
            for t in range(L):
                s = np.exp(dt[bi, t, h] * A[h]) * s + dt[bi, t, h] * np.outer(x[bi, t, h], Bm[bi, t])
                y[bi, t, h] = s @ Cm[bi, t] + Dv[h] * x[bi, t, h]
            hf[bi, h] = s
    return {"y": y, "h_final": hf}


def ssd_scan_bwd(x, dt_out, A, B, C, dy, D=None, h0=None, dh_final=None):
    """Gradients of the loss sum(dy * y) + sum(dh_final * h_final) of ssd_scan_fwd with
    respect to every input, by the reverse (adjoint) recurrence: with G = dLoss/dstate_t,
        G      += outer(dy_t, C_t)                      (y_t reads state_t)
        dC_t   += state_t^T dy_t,   dD += dy_t . x_t,   dx_t = D dy_t + dt_t G B_t
        dB_t   += dt_t G^T x_t
        ddt_t   = A a_t <G, state_{t-1}> + x_t^T G B_t,  dA += dt_t a_t <G, state_{t-1}>
        G       = a_t G                                  (a_t = exp(dt_t A))
    and dh0 = G after step 0.  dB and dC are summed over heads (one shared group).
    -> {"dx", "ddt" [batch, seqlen, heads], "dA" [heads], "dB", "dC", "dD", "dh0"}"""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt_out, np.float64)
    A = np.asarray(A, np.float64)
    Bm = np.asarray(B, np.float64)
    Cm = np.asarray(C, np.float64)
    dy = np.asarray(dy, np.float64)
    b, L, H, P = x.shape
    N = Bm.shape[-1]
    Dv = np.zeros(H) if D is None else np.asarray(D, np.float64)
    out = {"dx": np.zeros_like(x), "ddt": np.zeros((b, L, H)), "dA": np.zeros(H), "dB": np.zeros((b, L, N)),
           "dC": np.zeros((b, L, N)), "dD": np.zeros(H), "dh0": np.zeros((b, H, P, N))}
    for bi in range(b):
        for h in range(H):
            st = np.zeros((L + 1, P, N))  # st[t + 1] = state after step t, st[0] = h0
            if h0 is not None:
                st[0] = np.asarray(h0[bi, h], np.float64)
            for t in range(L):
                st[t + 1] = np.exp(dt[bi, t, h] * A[h]) * st[t] + dt[bi, t, h] * np.outer(x[bi, t, h], Bm[bi, t])
            G = np.zeros((P, N)) if dh_final is None else np.array(dh_final[bi, h], np.float64)
            for t in range(L - 1, -1, -1):
                a = np.exp(dt[bi, t, h] * A[h])
                G = G + np.outer(dy[bi, t, h], Cm[bi, t])
                out["dC"][bi, t] += st[t + 1].T @ dy[bi, t, h]
                out["dD"][h] += dy[bi, t, h] @ x[bi, t, h]
                out["dx"][bi, t, h] = Dv[h] * dy[bi, t, h] + dt[bi, t, h] * (G @ Bm[bi, t])
                out["dB"][bi, t] += dt[bi, t, h] * (G.T @ x[bi, t, h])
                gs = float(np.sum(G * st[t]))
                out["ddt"][bi, t, h] = A[h] * a * gs + x[bi, t, h] @ G @ Bm[bi, t]
                out["dA"][h] += dt[bi, t, h] * a * gs
                G = a * G
            out["dh0"][bi, h] = G
    return out
