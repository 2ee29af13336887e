"""fp64 oracle of the Mamba-3 projection preprocess and its adjoint -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library.

Source: the mamba3_preprocess_backward.slang page (oarust crate), which prints the
adjoint only.  Per token row, the projected row is laid out as
    [ z (inner) | x (inner) | B (bc_rows groups of state) | C (bc_rows x state) |
      dd_dt (heads) | dd_a (heads) | trap (heads) | angles (rope_angles) ]
and the adjoint (main() of the page) writes a row of the same layout:
  * z, x, trap and angle parts: the incoming gradients, copied;
  * each B and C group: the RMS-norm backward of that group, with
    inv_rms = 1 / sqrt(mean(v^2) + epsilon) over the group and dot = sum(g * v);
  * dd_dt: (dt gradient + adt gradient * a_token) * mask * (1 - exp(-softplus)),
    mask = softplus inside [dt_min, dt_max] (bounds included), raw dt = dd_dt + dt_bias;
    the same value is the row's dt_bias partial;
  * dd_a: adt gradient * dt * (heavy_tail > a_floor) * -heavy_tail'(raw a), with
    heavy_tail' = 1 for raw a >= 0 and 1 / (1 - raw a)^2 below.
The functions the page imports but does not print are read as follows (the forward
whose derivative the adjoint is; the pins check that the adjoint is that derivative):
  * ssm_rms_norm_backward(v, g, inv, dot, n) = inv * g - v * inv^3 * dot / n, the
    derivative of the weightless RMS norm v * inv_rms(v);
  * heavy_tail(r) = 1 + r for r >= 0 and 1 / (1 - r) below: positive, continuous and
    with the printed derivative (the constant is fixed by continuity at 0 and by a
    tail that tends to 0, so that a positive floor a_floor is meaningful);
  * a_token = -max(heavy_tail, a_floor) (a negative decay rate: its derivative is
    -heavy_tail' where heavy_tail > a_floor, else 0, as the printed gradient has);
  * dt = clamp(softplus(raw dt), dt_min, dt_max), adt = a_token * dt.
d_dt_bias sums the row partials over rows in ascending row order.
"""
from __future__ import annotations

import numpy as np


def layout(inner, state, heads, rope_angles, bc_rows):
    """offsets of the parts of one projected row, and the row width"""
    bcw = bc_rows * state
    o = {"z": 0, "x": inner, "B": 2 * inner, "C": 2 * inner + bcw}
    o["dd_dt"] = o["C"] + bcw
    o["dd_a"] = o["dd_dt"] + heads
    o["trap"] = o["dd_a"] + heads
    o["angles"] = o["trap"] + heads
    o["width"] = o["angles"] + rope_angles
    return o


def softplus(r):
    return np.maximum(r, 0.0) + np.log1p(np.exp(-np.abs(r)))


def heavy_tail(r):
    return np.where(r >= 0.0, 1.0 + np.maximum(r, 0.0), 1.0 / (1.0 - np.minimum(r, 0.0)))


def heavy_tail_grad(r):
    return np.where(r >= 0.0, 1.0, 1.0 / (1.0 - np.minimum(r, 0.0)) ** 2)


def preprocess_fwd(projected, dt_bias, inner, state, heads, rope_angles, bc_rows, epsilon, dt_min, dt_max,
                   a_floor):
    """The forward preprocess read from the adjoint: per row z, x, normalised B and C
    ([rows, bc_rows, state]), dt, adt ([rows, heads]), trap, angles."""
    p = np.asarray(projected, np.float64)
    o = layout(inner, state, heads, rope_angles, bc_rows)
    rows = p.shape[0]
    assert p.shape == (rows, o["width"])
    out = {"z": p[:, o["z"]:o["z"] + inner].copy(), "x": p[:, o["x"]:o["x"] + inner].copy()}
    for name in ("B", "C"):
        v = p[:, o[name]:o[name] + bc_rows * state].reshape(rows, bc_rows, state)
        inv = 1.0 / np.sqrt(np.mean(v * v, axis=2, keepdims=True) + epsilon)
        out[name] = v * inv
    sp = softplus(p[:, o["dd_dt"]:o["dd_dt"] + heads] + np.asarray(dt_bias, np.float64)[None, :])
    dt = np.clip(sp, dt_min, dt_max)
    a_token = -np.maximum(heavy_tail(p[:, o["dd_a"]:o["dd_a"] + heads]), a_floor)
    out["dt"] = dt
    out["adt"] = a_token * dt
    out["trap"] = p[:, o["trap"]:o["trap"] + heads].copy()
    out["angles"] = p[:, o["angles"]:o["angles"] + rope_angles].copy()
    return out


def preprocess_bwd(projected, dt_bias, grads, inner, state, heads, rope_angles, bc_rows, epsilon, dt_min, dt_max,
                   a_floor):
    """The adjoint, following the page's steps row by row.

    grads: dict with z [rows, inner], x [rows, inner], B and C [rows, bc_rows*state],
    dt, adt, trap [rows, heads], angles [rows, rope_angles].
    Returns {"projected": gradient row per token, "dt_bias_partial": [rows, heads],
    "d_dt_bias": [heads]}.
    """
    p = np.asarray(projected, np.float64)
    bias = np.asarray(dt_bias, np.float64)
    g = {k: np.asarray(v, np.float64) for k, v in grads.items()}
    o = layout(inner, state, heads, rope_angles, bc_rows)
    rows = p.shape[0]
    out = np.zeros((rows, o["width"]))
    partial = np.zeros((rows, heads))
    for row in range(rows):
        pr = p[row]
        for name, gk in (("B", "B"), ("C", "C")):
            for grp in range(bc_rows):
                lo = o[name] + grp * state
                v = pr[lo:lo + state]
                gv = g[gk][row, grp * state:(grp + 1) * state]
                inv = 1.0 / np.sqrt(np.sum(v * v) / state + epsilon)
                dot = np.sum(gv * v)
                out[row, lo:lo + state] = inv * gv - v * inv ** 3 * dot / state
        out[row, o["z"]:o["z"] + inner] = g["z"][row]
        out[row, o["x"]:o["x"] + inner] = g["x"][row]
        for h in range(heads):
            raw_dt = pr[o["dd_dt"] + h] + bias[h]
            sp = float(softplus(raw_dt))
            dt = min(max(sp, dt_min), dt_max)
            raw_a = pr[o["dd_a"] + h]
            ht = float(heavy_tail(raw_a))
            a_token = -max(ht, a_floor)
            total = g["dt"][row, h] + g["adt"][row, h] * a_token
            mask = 1.0 if (dt_min <= sp <= dt_max) else 0.0
            rdt = total * mask * (1.0 - np.exp(-sp))
            out[row, o["dd_dt"] + h] = rdt
            partial[row, h] = rdt
            ht_mask = 1.0 if ht > a_floor else 0.0
            out[row, o["dd_a"] + h] = g["adt"][row, h] * dt * ht_mask * -float(heavy_tail_grad(raw_a))
            out[row, o["trap"] + h] = g["trap"][row, h]
        out[row, o["angles"]:o["angles"] + rope_angles] = g["angles"][row]
    d_dt_bias = np.zeros(heads)
    for row in range(rows):  # ascending row order
        d_dt_bias += partial[row]
    return {"projected": out, "dt_bias_partial": partial, "d_dt_bias": d_dt_bias}
