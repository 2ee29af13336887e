"""fp64 oracle of the Mamba-2 SSD chunk cumsum and its ordered backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library.

Source: deterministic_backward.py (pretraining_mamba2_outer), ordered_cumsum.  Its
arguments fix what the chunk cumsum computes and what its backward returns:
  forward  (dt [batch, seqlen, heads], A [heads], dt_bias [heads] optional,
            dt_softplus, dt_limit = (dt_min, dt_max), chunk width W):
    dt_out[b, h, c, l]    = clamp(g(dt[b, c*W + l, h] + dt_bias[h]), dt_min, dt_max)
                            (g = softplus when dt_softplus, else the identity;
                             0 for positions past the end of the sequence)
    dA_cumsum[b, h, c, l] = sum_{l' <= l} dt_out[b, h, c, l'] * A[h]   (inside chunk c)
  backward (ddA = dLoss/dA_cumsum, ddt_out = dLoss/dt_out, both [batch, heads,
            chunks, W]):
    ddt_out_total         = ddt_out + A * sum_{l' >= l} ddA[.., l']
    ddt[b, t, h]          = ddt_out_total * mask * g'(dt + dt_bias)
                            (mask: the value before the clamp lies in [dt_min, dt_max])
    dA[h]                 = sum over (b, c) in lexical order of the per-(b, c) partial
                            sum_l dt_out * sum_{l' >= l} ddA[.., l']
    d_dt_bias[h]          = the same ordered sum of per-(b, c) partials of ddt
The page accumulates one partial per (batch, chunk) call "in lexical order" in fp32
(dA.add_, db.add_); here every partial and sum is fp64, added in the same order.
Plainest readings where the page is silent: the clamp mask includes its bounds (as the
Mamba-3 page's dt mask does), and dt_limit = (0, inf) is no clamp.
"""
from __future__ import annotations

import numpy as np


def _g(r, softplus):
    if softplus:
        return np.maximum(r, 0.0) + np.log1p(np.exp(-np.abs(r)))
    return r


def _g_prime(r, softplus):
    if softplus:
        return np.where(r >= 0, 1.0 / (1.0 + np.exp(-np.abs(r))), np.exp(-np.abs(r)) / (1.0 + np.exp(-np.abs(r))))
    return np.ones_like(r)


def chunk_cumsum_fwd(dt, A, dt_bias, chunk, dt_softplus=True, dt_min=0.0, dt_max=float("inf")):
    """-> (dA_cumsum, dt_out), both [batch, heads, chunks, chunk]"""
    dt = np.asarray(dt, np.float64)
    b, L, H = dt.shape
    A = np.asarray(A, np.float64)
    bias = np.zeros(H) if dt_bias is None else np.asarray(dt_bias, np.float64)
    nc = (L + chunk - 1) // chunk
    dt_out = np.zeros((b, H, nc, chunk))
    dA_cs = np.zeros((b, H, nc, chunk))
    for bi in range(b):
        for h in range(H):
            for c in range(nc):
                acc = 0.0
                for l in range(chunk):
                    t = c * chunk + l
                    if t < L:
                        v = float(_g(dt[bi, t, h] + bias[h], dt_softplus))
                        v = min(max(v, dt_min), dt_max)
                    else:
                        v = 0.0
                    dt_out[bi, h, c, l] = v
                    acc += v * A[h]
                    dA_cs[bi, h, c, l] = acc
    return dA_cs, dt_out


def chunk_cumsum_bwd(ddA, ddt_out, dt, A, dt_bias, chunk, dt_softplus=True, dt_min=0.0, dt_max=float("inf")):
    """-> {"ddt" [batch, seqlen, heads], "dA" [heads], "d_dt_bias" [heads],
    "dA_partial", "db_partial" [batch, chunks, heads]}"""
    ddA = np.asarray(ddA, np.float64)
    ddt_out = np.asarray(ddt_out, np.float64)
    dt = np.asarray(dt, np.float64)
    b, L, H = dt.shape
    A = np.asarray(A, np.float64)
    bias = np.zeros(H) if dt_bias is None else np.asarray(dt_bias, np.float64)
    nc = (L + chunk - 1) // chunk
    _, dt_out = chunk_cumsum_fwd(dt, A, dt_bias, chunk, dt_softplus, dt_min, dt_max)
    ddt = np.zeros((b, L, H))
    pa = np.zeros((b, nc, H))
    pb = np.zeros((b, nc, H))
    for bi in range(b):
        for c in range(nc):
            for h in range(H):
                rev = 0.0
                for l in range(chunk - 1, -1, -1):
                    rev += ddA[bi, h, c, l]  # sum over l' >= l
                    t = c * chunk + l
                    pa[bi, c, h] += dt_out[bi, h, c, l] * rev
                    if t >= L:
                        continue
                    total = ddt_out[bi, h, c, l] + A[h] * rev
                    r = dt[bi, t, h] + bias[h]
                    pre = float(_g(r, dt_softplus))
                    mask = 1.0 if (dt_min <= pre <= dt_max) else 0.0
                    v = total * mask * float(_g_prime(np.array(r), dt_softplus))
                    ddt[bi, t, h] = v
                    pb[bi, c, h] += v
    dA = np.zeros(H)
    db = np.zeros(H)
    for bi in range(b):  # lexical (batch, chunk) order
        for c in range(nc):
            dA += pa[bi, c]
            db += pb[bi, c]
    return {"ddt": ddt, "dA": dA, "d_dt_bias": db, "dA_partial": pa, "db_partial": pb}
