"""Pins of the Mamba-3 preprocess-adjoint oracle against facts that do not come from it.

* central differences: the adjoint equals the gradient of
  L = sum over outputs of (incoming gradient * forward output) with respect to every
  element of the projected rows and of dt_bias (inputs kept away from the kinks of
  the clamp, the floor and heavy_tail);
* heavy_tail: continuous with slope 1 on both sides of 0, positive, tail -> 0;
* RMS norm of a constant group: closed-form value and gradient;
* masks: steps clamped by [dt_min, dt_max] and decay rates below a_floor pass no
  gradient; the copied parts are the incoming gradients exactly;
* d_dt_bias is the row sum of the per-row partials.
"""
import numpy as np
import pytest

from oracle import mamba3_oracle as M


def problem(rng, rows=4, inner=6, state=5, heads=3, angles=4, bc=2):
    o = M.layout(inner, state, heads, angles, bc)
    p = rng.standard_normal((rows, o["width"]))
    p[:, o["dd_dt"]:o["dd_dt"] + heads] *= 2.0
    bias = rng.uniform(-2.0, 0.5, heads)
    g = {"z": rng.standard_normal((rows, inner)), "x": rng.standard_normal((rows, inner)),
         "B": rng.standard_normal((rows, bc * state)), "C": rng.standard_normal((rows, bc * state)),
         "dt": rng.standard_normal((rows, heads)), "adt": rng.standard_normal((rows, heads)),
         "trap": rng.standard_normal((rows, heads)), "angles": rng.standard_normal((rows, angles))}
    return dict(p=p, bias=bias, g=g, dims=(inner, state, heads, angles, bc))


def loss(prob, p, bias, eps, lo, hi, floor):
    inner, state, heads, angles, bc = prob["dims"]
    f = M.preprocess_fwd(p, bias, inner, state, heads, angles, bc, eps, lo, hi, floor)
    rows = p.shape[0]
    g = prob["g"]
    total = 0.0
    for k in ("z", "x", "dt", "adt", "trap", "angles"):
        total += float(np.sum(g[k] * f[k]))
    for k in ("B", "C"):
        total += float(np.sum(g[k] * f[k].reshape(rows, bc * state)))
    return total


def kink_free_bounds(prob, gap=1e-3):
    """clamp bounds at quantiles of softplus and a floor at a quantile of heavy_tail,
    each moved until no element is within `gap` (relative) of it"""
    inner, state, heads, angles, bc = prob["dims"]
    o = M.layout(inner, state, heads, angles, bc)
    sp = M.softplus(prob["p"][:, o["dd_dt"]:o["dd_dt"] + heads] + prob["bias"][None]).ravel()
    ht = M.heavy_tail(prob["p"][:, o["dd_a"]:o["dd_a"] + heads]).ravel()

    def clear(v, x):
        for _ in range(1000):
            if np.min(np.abs(v - x)) > gap * x:
                return x
            x *= 1.0 + 2 * gap
        raise AssertionError("no kink-free bound")

    lo = clear(sp, float(np.quantile(sp, 0.25)))
    hi = clear(sp, float(np.quantile(sp, 0.8)))
    floor = clear(ht, float(np.quantile(ht, 0.3)))
    return lo, hi, floor


@pytest.mark.parametrize("seed", [1, 2])
def test_adjoint_matches_central_differences(seed):
    rng = np.random.default_rng(300 + seed)
    prob = problem(rng)
    inner, state, heads, angles, bc = prob["dims"]
    o = M.layout(inner, state, heads, angles, bc)
    # keep raw a away from 0 (heavy_tail's second derivative jumps there)
    a = prob["p"][:, o["dd_a"]:o["dd_a"] + heads]
    a[np.abs(a) < 1e-2] += 0.05
    eps = 1e-3
    lo, hi, floor = kink_free_bounds(prob)
    r = M.preprocess_bwd(prob["p"], prob["bias"], prob["g"], inner, state, heads, angles, bc, eps, lo, hi, floor)
    p, bias = prob["p"], prob["bias"]
    fd = np.zeros_like(p)
    for idx in np.ndindex(p.shape):
        h = 1e-6 * max(1.0, abs(p[idx]))
        up, dn = p.copy(), p.copy()
        up[idx] += h
        dn[idx] -= h
        fd[idx] = (loss(prob, up, bias, eps, lo, hi, floor) - loss(prob, dn, bias, eps, lo, hi, floor)) / (2 * h)
    np.testing.assert_allclose(r["projected"], fd, rtol=1e-6, atol=1e-6 * max(1.0, np.abs(fd).max()))
    fdb = np.zeros_like(bias)
    for j in range(heads):
        h = 1e-6
        up, dn = bias.copy(), bias.copy()
        up[j] += h
        dn[j] -= h
        fdb[j] = (loss(prob, p, up, eps, lo, hi, floor) - loss(prob, p, dn, eps, lo, hi, floor)) / (2 * h)
    np.testing.assert_allclose(r["d_dt_bias"], fdb, rtol=1e-6, atol=1e-7)
    # the clamps and the floor were active in this problem
    sp = M.softplus(p[:, o["dd_dt"]:o["dd_dt"] + heads] + bias[None])
    assert np.any(sp < lo) and np.any(sp > hi)
    assert np.any(M.heavy_tail(p[:, o["dd_a"]:o["dd_a"] + heads]) < floor)


def test_heavy_tail_shape():
    r = np.array([-1e6, -10.0, -1e-9, 0.0, 1e-9, 3.0])
    ht = M.heavy_tail(r)
    assert ht[3] == 1.0 and abs(ht[2] - 1.0) < 1e-8 and abs(ht[4] - 1.0) < 1e-8
    assert np.all(ht > 0.0) and ht[0] < 2e-6
    np.testing.assert_allclose(ht[1], 1.0 / 11.0)
    np.testing.assert_allclose(ht[5], 4.0)
    # slope 1 on both sides of 0, from finite differences of the function itself
    h = 1e-7
    for x in (-1e-3, 1e-3):
        fd = (M.heavy_tail(np.array(x + h)) - M.heavy_tail(np.array(x - h))) / (2 * h)
        np.testing.assert_allclose(fd, M.heavy_tail_grad(np.array(x)), rtol=1e-6)
    np.testing.assert_allclose(M.heavy_tail_grad(np.array([-1e-12, 0.0])), [1.0, 1.0], rtol=1e-9)


def test_rms_norm_of_a_constant_group():
    """v = c on a group of n: v_hat = c / sqrt(c^2 + eps); with incoming gradient 1 on
    every element the gradient is eps / (c^2 + eps)^(3/2)."""
    inner, state, heads, angles, bc = 2, 8, 1, 2, 1
    o = M.layout(inner, state, heads, angles, bc)
    c, eps = 0.7, 1e-2
    p = np.zeros((1, o["width"]))
    p[0, o["B"]:o["B"] + state] = c
    p[0, o["C"]:o["C"] + state] = -c
    f = M.preprocess_fwd(p, np.zeros(1), inner, state, heads, angles, bc, eps, 0.0, np.inf, 0.0)
    np.testing.assert_allclose(f["B"], c / np.sqrt(c * c + eps))
    np.testing.assert_allclose(f["C"], -c / np.sqrt(c * c + eps))
    g = {"z": np.zeros((1, inner)), "x": np.zeros((1, inner)), "B": np.ones((1, state)),
         "C": np.ones((1, state)), "dt": np.zeros((1, 1)), "adt": np.zeros((1, 1)),
         "trap": np.zeros((1, 1)), "angles": np.zeros((1, angles))}
    r = M.preprocess_bwd(p, np.zeros(1), g, inner, state, heads, angles, bc, eps, 0.0, np.inf, 0.0)
    want = eps / (c * c + eps) ** 1.5
    np.testing.assert_allclose(r["projected"][0, o["B"]:o["B"] + state], want, rtol=1e-12)
    np.testing.assert_allclose(r["projected"][0, o["C"]:o["C"] + state], want, rtol=1e-12)


def test_masks_and_copied_parts():
    rng = np.random.default_rng(310)
    prob = problem(rng, rows=3)
    inner, state, heads, angles, bc = prob["dims"]
    o = M.layout(inner, state, heads, angles, bc)
    p, bias, g = prob["p"], prob["bias"], prob["g"]
    # every softplus above dt_max, every heavy_tail below a_floor
    r = M.preprocess_bwd(p, bias, g, inner, state, heads, angles, bc, 1e-5, 1e-9, 2e-9, 1e9)
    assert np.all(r["projected"][:, o["dd_dt"]:o["dd_dt"] + heads] == 0.0)
    assert np.all(r["projected"][:, o["dd_a"]:o["dd_a"] + heads] == 0.0)
    assert np.all(r["d_dt_bias"] == 0.0)
    for part, key, width in (("z", "z", inner), ("x", "x", inner), ("trap", "trap", heads),
                             ("angles", "angles", angles)):
        assert np.array_equal(r["projected"][:, o[part]:o[part] + width], g[key]), part
    np.testing.assert_allclose(r["d_dt_bias"], r["dt_bias_partial"].sum(axis=0), rtol=1e-15)
