"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each check would fail under a plausible mistake in the oracle (a dropped term,
a wrong sign or index, readout from the stale state, a transposed operand):
  * closed-form geometric sum for constant inputs (long L, random h0, gated);
  * brute-force unrolled product form at L <= 8 (independent O(L^2) code);
  * the L=1 scan equals the separately written single-step update;
  * zero input and zero state give exactly zero;
  * composition: scan(L1+L2) == scan(L2, h0 = h_final(scan(L1)));
  * linearity in x (ungated, h0 = 0);
  * hand-derived worked examples (tests/golden/hand_cases.json);
  * backward: central finite differences of sum(dy*y) (and of sum(dy*y) +
    sum(dh_final*h_final), giving dh0) for every input and
    parameter element, gated and ungated; special case C = 0; an adjoint
    (directional-derivative) identity; thread-count independence;
  * a backward split in two segments (dh0 of the second part as dh_final of the
    first) equals the backward of the whole sequence;
  * step-size clamp: central differences with steps clamped below, above and not
    at all (clamped steps pass no gradient to delta_raw); dt_min = dt_max = c gives
    the constant-step closed form whatever delta_raw is; a clamp that never binds
    changes nothing; the clamped L=1 scan equals the clamped step.
The oracle's scalar helpers are pinned to library routines (numpy logaddexp,
the logistic function) and to the softplus identity sigma(r) = 1 - exp(-softplus(r)).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from selective_state_space_03_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def softplus_ref(r):
    return np.logaddexp(0.0, r)  # library routine: log(exp(0) + exp(r))


def silu_ref(z):
    return z / (1.0 + np.exp(-z))


def rand_problem(rng, b, l, d, n, gated=True, h0=True, dscale=1.0):
    p = {
        "x": rng.standard_normal((b, l, d)),
        "delta_raw": rng.standard_normal((b, l, d)) * dscale,
        "B": rng.standard_normal((b, l, n)),
        "C": rng.standard_normal((b, l, n)),
        "A_log": rng.standard_normal((d, n)) * 0.5,
        "D": rng.standard_normal(d),
        "dt_bias": rng.standard_normal(d) * 0.5,
        "z": rng.standard_normal((b, l, d)) if gated else None,
        "h0": rng.standard_normal((b, d, n)) if h0 else None,
    }
    return p


def run_fwd(p, **kw):
    return oracle.fwd(p["x"], p["delta_raw"], p["B"], p["C"], p["A_log"], D=p["D"],
                      dt_bias=p["dt_bias"], z=p.get("z"), h0=p.get("h0"), **kw)


def run_bwd(p, dy, **kw):
    return oracle.bwd(p["x"], p["delta_raw"], p["B"], p["C"], p["A_log"], dy, D=p["D"],
                      dt_bias=p["dt_bias"], z=p.get("z"), h0=p.get("h0"), **kw)


# ---------------------------------------------------------------- scalar helpers

def test_scalar_helpers_match_library_routines():
    for r in np.linspace(-30, 30, 241):
        sp = oracle.softplus(r)
        assert sp == pytest.approx(float(softplus_ref(r)), rel=1e-14, abs=1e-300)
        sg = oracle.sigmoid(r)
        assert sg == pytest.approx(1.0 / (1.0 + math.exp(-r)), rel=1e-14)
        # softplus identity used by the dt adjoint: sigmoid(r) = 1 - exp(-softplus(r))
        assert sg == pytest.approx(-math.expm1(-sp), rel=1e-12)
        assert oracle.silu(r) == pytest.approx(float(silu_ref(r)), rel=1e-14, abs=1e-300)
        h = 1e-5
        fd = (oracle.silu(r + h) - oracle.silu(r - h)) / (2 * h)
        assert oracle.silu_grad(r) == pytest.approx(fd, rel=1e-7, abs=1e-9)
    assert oracle.softplus(800.0) == 800.0
    assert oracle.softplus(-800.0) == 0.0


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("L", [1, 7, 256, 4096])
def test_closed_form_geometric_sum(gated, L):
    """Constant inputs over time: h_t = a^(t+1) h0 + u (1 - a^(t+1)) / (1 - a)."""
    rng = np.random.default_rng(7 + L)
    b, d, n = 2, 3, 5
    xc = rng.standard_normal((b, d))
    rc = rng.standard_normal((b, d)) - 2.0
    zc = rng.standard_normal((b, d))
    Bc = rng.standard_normal((b, n))
    Cc = rng.standard_normal((b, n))
    A_log = np.log(rng.uniform(0.05, 3.0, (d, n)))
    Dsk = rng.standard_normal(d)
    bias = 0.3 * rng.standard_normal(d)
    h0 = rng.standard_normal((b, d, n))
    rep = lambda a: np.repeat(a[:, None, :], L, axis=1)
    res = oracle.fwd(rep(xc), rep(rc), rep(Bc), rep(Cc), A_log, D=Dsk, dt_bias=bias,
                     z=rep(zc) if gated else None, h0=h0)
    delta = softplus_ref(rc + bias[None, :])                     # [b, d]
    A = -np.exp(A_log)                                            # [d, n]
    a = np.exp(delta[:, :, None] * A[None])                       # [b, d, n]
    u = delta[:, :, None] * Bc[:, None, :] * xc[:, :, None]       # [b, d, n]
    t = np.arange(1, L + 1)[None, :, None, None]                  # powers t+1
    ak = a[:, None] ** t                                          # [b, L, d, n]
    h = ak * h0[:, None] + u[:, None] * (1 - ak) / (1 - a[:, None])
    s = np.einsum("bldn,bn->bld", h, Cc) + Dsk[None, None, :] * xc[:, None, :]
    y = s * silu_ref(zc)[:, None, :] if gated else s
    np.testing.assert_allclose(res["y"], y, rtol=1e-11, atol=1e-12 * np.abs(y).max())
    np.testing.assert_allclose(res["h_final"], h[:, -1], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 3, 5, 8])
def test_bruteforce_unroll(L):
    """h_t = (prod_{s<=t} a_s) h0 + sum_s (prod_{s<r<=t} a_r) u_s, written out in O(L^2)."""
    rng = np.random.default_rng(100 + L)
    b, d, n = 2, 4, 3
    p = rand_problem(rng, b, l=L, d=d, n=n)
    res = run_fwd(p)
    A = -np.exp(p["A_log"])
    y = np.zeros((b, L, d))
    hT = np.zeros((b, d, n))
    for bi in range(b):
        for di in range(d):
            delta = [softplus_ref(p["delta_raw"][bi, t, di] + p["dt_bias"][di]) for t in range(L)]
            for t in range(L):
                hv = np.zeros(n)
                for nn in range(n):
                    decay = 1.0
                    for r in range(t + 1):
                        decay *= math.exp(delta[r] * A[di, nn])
                    acc = decay * p["h0"][bi, di, nn]
                    for s_ in range(t + 1):
                        prod = 1.0
                        for r in range(s_ + 1, t + 1):
                            prod *= math.exp(delta[r] * A[di, nn])
                        acc += prod * delta[s_] * p["B"][bi, s_, nn] * p["x"][bi, s_, di]
                    hv[nn] = acc
                s = float(np.dot(p["C"][bi, t], hv)) + p["D"][di] * p["x"][bi, t, di]
                y[bi, t, di] = s * silu_ref(p["z"][bi, t, di])
                if t == L - 1:
                    hT[bi, di] = hv
    np.testing.assert_allclose(res["y"], y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res["h_final"], hT, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("gated", [False, True])
def test_scan_of_length_one_equals_step(gated):
    rng = np.random.default_rng(3)
    b, d, n = 4, 9, 16
    p = rand_problem(rng, b, 1, d, n, gated=gated)
    res = run_fwd(p)
    st = oracle.step(p["h0"], p["x"][:, 0], p["delta_raw"][:, 0], p["B"][:, 0], p["C"][:, 0], p["A_log"],
                     D=p["D"], dt_bias=p["dt_bias"], z=p["z"][:, 0] if gated else None)
    np.testing.assert_allclose(st["y"], res["y"][:, 0], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(st["state"], res["h_final"], rtol=1e-15, atol=1e-15)


def test_zero_input_zero_state_is_exactly_zero():
    w = W.WORKLOADS["fwd_b8_l2048_d1536"]
    inp = W.make_inputs(w, batch=2, seqlen=300, dim=20)
    x0 = np.zeros_like(inp["x"])
    res = oracle.fwd(x0, inp["delta_raw"], inp["B"], inp["C"], inp["A_log"], D=inp["D"],
                     dt_bias=inp["dt_bias"], z=inp["z"])
    assert np.all(res["y"] == 0.0) and np.all(res["h_final"] == 0.0)


def test_composition_of_segments():
    rng = np.random.default_rng(11)
    b, d, n, L1, L2 = 2, 6, 8, 37, 91
    p = rand_problem(rng, b, L1 + L2, d, n)
    full = run_fwd(p)
    p1 = {k: (v[:, :L1] if k in ("x", "delta_raw", "B", "C", "z") else v) for k, v in p.items()}
    first = run_fwd(p1)
    p2 = {k: (v[:, L1:] if k in ("x", "delta_raw", "B", "C", "z") else v) for k, v in p.items()}
    p2["h0"] = first["h_final"]
    second = run_fwd(p2)
    np.testing.assert_allclose(np.concatenate([first["y"], second["y"]], 1), full["y"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(second["h_final"], full["h_final"], rtol=1e-13, atol=1e-13)


def test_linearity_in_x():
    rng = np.random.default_rng(5)
    b, l, d, n = 2, 50, 5, 4
    p = rand_problem(rng, b, l, d, n, gated=False, h0=False)
    x1, x2 = rng.standard_normal((2, b, l, d))
    al, be = 0.7, -1.3
    y = lambda x: oracle.fwd(x, p["delta_raw"], p["B"], p["C"], p["A_log"], D=p["D"], dt_bias=p["dt_bias"])["y"]
    np.testing.assert_allclose(y(al * x1 + be * x2), al * y(x1) + be * y(x2), rtol=1e-12, atol=1e-12)


def test_thread_count_does_not_change_forward():
    w = W.WORKLOADS["fwd_b8_l2048_d1536"]
    inp = W.make_inputs(w, batch=2, seqlen=64, dim=33)
    args = (inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"])
    kw = dict(D=inp["D"], dt_bias=inp["dt_bias"], z=inp["z"])
    r1 = oracle.fwd(*args, nthreads=1, **kw)
    r5 = oracle.fwd(*args, nthreads=5, **kw)
    assert np.array_equal(r1["y"], r5["y"]) and np.array_equal(r1["h_final"], r5["h_final"])


# ---------------------------------------------------------------- golden hand cases

def _ev(v):
    env = {"ln2": math.log(2.0), "e": math.e, "log": math.log, "exp": math.exp, "__builtins__": {}}
    if isinstance(v, list):
        return [_ev(u) for u in v]
    if isinstance(v, str):
        return eval(v, env)  # expressions from the committed fixture file only
    return float(v)


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    inp = {k: np.array(_ev(v), dtype=np.float64) for k, v in case["inputs"].items()}
    args = (inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"])
    kw = dict(D=inp.get("D"), dt_bias=inp.get("dt_bias"), z=inp.get("z"), h0=inp.get("h0"))
    if "fwd" in case:
        res = oracle.fwd(*args, **kw)
        for k, v in case["fwd"].items():
            np.testing.assert_allclose(res[k], np.array(_ev(v)), rtol=1e-14, atol=1e-15, err_msg=k)
    if "bwd" in case:
        res = oracle.bwd(*args, inp["dy"], **kw)
        for k, v in case["bwd"].items():
            np.testing.assert_allclose(res[k], np.array(_ev(v)), rtol=1e-14, atol=1e-15, err_msg=k)


# ---------------------------------------------------------------- backward pins

GRAD_OF = {"x": "dx", "delta_raw": "ddelta_raw", "z": "dz", "B": "dB", "C": "dC",
           "A_log": "dA_log", "D": "dD", "dt_bias": "d_dt_bias"}


@pytest.mark.parametrize("gated", [False, True])
def test_backward_matches_central_differences(gated):
    rng = np.random.default_rng(21 if gated else 22)
    b, l, d, n = 2, 5, 3, 2
    p = rand_problem(rng, b, l, d, n, gated=gated, h0=True)
    dy = rng.standard_normal((b, l, d))
    g = run_bwd(p, dy)
    loss = lambda q: float(np.sum(dy * run_fwd(q)["y"]))
    for name, gname in GRAD_OF.items():
        if p.get(name) is None:
            continue
        base = p[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hstep = 1e-6 * max(1.0, abs(base[idx]))
            q = dict(p)
            up = base.copy(); up[idx] += hstep
            dn = base.copy(); dn[idx] -= hstep
            q[name] = up
            lp = loss(q)
            q[name] = dn
            lm = loss(q)
            fd[idx] = (lp - lm) / (2 * hstep)
        scale = max(1.0, np.abs(fd).max())
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-6 * scale, err_msg=name)


def test_backward_adjoint_identity():
    """<dy, J v> (directional derivative of y) equals <J^T dy, v> over all inputs at once."""
    rng = np.random.default_rng(31)
    b, l, d, n = 1, 64, 16, 4
    p = rand_problem(rng, b, l, d, n, gated=True, h0=False)
    dy = rng.standard_normal((b, l, d))
    g = run_bwd(p, dy)
    v = {k: rng.standard_normal(p[k].shape) for k in GRAD_OF}
    eps = 1e-6
    qp = {k: (p[k] + eps * v[k] if k in v else p[k]) for k in p}
    qm = {k: (p[k] - eps * v[k] if k in v else p[k]) for k in p}
    jv = (run_fwd(qp)["y"] - run_fwd(qm)["y"]) / (2 * eps)
    lhs = float(np.sum(dy * jv))
    rhs = sum(float(np.sum(g[GRAD_OF[k]] * v[k])) for k in v)
    assert lhs == pytest.approx(rhs, rel=1e-7)


def test_backward_with_zero_C():
    """C = 0 leaves y = D x silu(z): only dx, dz, dD (and dC) can be nonzero."""
    rng = np.random.default_rng(41)
    b, l, d, n = 2, 30, 4, 3
    p = rand_problem(rng, b, l, d, n, gated=True, h0=True)
    p["C"] = np.zeros_like(p["C"])
    dy = rng.standard_normal((b, l, d))
    g = run_bwd(p, dy)
    gate = silu_ref(p["z"])
    gg = dy * gate
    np.testing.assert_allclose(g["dx"], gg * p["D"][None, None, :], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g["dD"], np.sum(gg * p["x"], axis=(0, 1)), rtol=1e-12)
    for k in ("dB", "dA_log", "d_dt_bias", "ddelta_raw"):
        assert np.all(g[k] == 0.0), k
    # dC_t[n] = sum_d g_t h_t[n] with h from the forward scan
    h = np.zeros((b, l, d, n))
    for t in range(l):
        pp = {kk: (vv[:, : t + 1] if kk in ("x", "delta_raw", "B", "C", "z") else vv) for kk, vv in p.items()}
        h[:, t] = run_fwd(pp)["h_final"]
    np.testing.assert_allclose(g["dC"], np.einsum("bld,bldn->bln", gg, h), rtol=1e-12, atol=1e-13)


def test_backward_thread_count_consistent():
    w = W.WORKLOADS["fwdbwd_b4_l2048_d2048"]
    inp = W.make_inputs(w, batch=2, seqlen=40, dim=12)
    args = (inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"], inp["dy"])
    kw = dict(D=inp["D"], dt_bias=inp["dt_bias"], z=inp["z"])
    g1 = oracle.bwd(*args, nthreads=1, **kw)
    g4 = oracle.bwd(*args, nthreads=4, **kw)
    for k in g1:
        if g1[k] is None:
            continue
        if k in ("dB", "dC"):
            np.testing.assert_allclose(g1[k], g4[k], rtol=1e-13, atol=1e-13)
        else:
            assert np.array_equal(g1[k], g4[k]), k


# ------------------------------------------- sequences carried across segments

def _fd_grads(p, loss, names):
    """central differences of a scalar loss for every element of the named inputs"""
    out = {}
    for name in names:
        base = p[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hstep = 1e-6 * max(1.0, abs(base[idx]))
            q = dict(p)
            up = base.copy(); up[idx] += hstep
            dn = base.copy(); dn[idx] -= hstep
            q[name] = up
            lp = loss(q)
            q[name] = dn
            lm = loss(q)
            fd[idx] = (lp - lm) / (2 * hstep)
        out[name] = fd
    return out


@pytest.mark.parametrize("gated", [False, True])
def test_backward_with_final_state_gradient_matches_central_differences(gated):
    """Loss sum(dy*y) + sum(dh_final*h_final): every gradient, and dh0, against central
    differences (initial_states / dfinal_states of deterministic_backward.py)."""
    rng = np.random.default_rng(61 if gated else 62)
    b, l, d, n = 2, 5, 3, 2
    p = rand_problem(rng, b, l, d, n, gated=gated, h0=True)
    dy = rng.standard_normal((b, l, d))
    dhf = rng.standard_normal((b, d, n))
    g = run_bwd(p, dy, dh_final=dhf)

    def loss(q):
        r = run_fwd(q)
        return float(np.sum(dy * r["y"]) + np.sum(dhf * r["h_final"]))

    names = [k for k in list(GRAD_OF) + ["h0"] if p.get(k) is not None]
    fd = _fd_grads(p, loss, names)
    for name in names:
        gname = GRAD_OF.get(name, "dh0")
        scale = max(1.0, np.abs(fd[name]).max())
        np.testing.assert_allclose(g[gname], fd[name], rtol=1e-6, atol=1e-6 * scale, err_msg=name)


def test_backward_composes_over_segments():
    """Backward of a whole sequence = backward of its second part (started from the
    first part's final state) followed by backward of the first part with the second
    part's dh0 as its dh_final: per-step gradients match, parameter gradients add."""
    rng = np.random.default_rng(63)
    b, d, n, L1, L2 = 2, 5, 4, 23, 41
    p = rand_problem(rng, b, L1 + L2, d, n, gated=True, h0=True)
    dy = rng.standard_normal((b, L1 + L2, d))
    dhf = rng.standard_normal((b, d, n))
    full = run_bwd(p, dy, dh_final=dhf)
    seq = ("x", "delta_raw", "B", "C", "z")
    p1 = {k: (v[:, :L1] if k in seq else v) for k, v in p.items()}
    p2 = {k: (v[:, L1:] if k in seq else v) for k, v in p.items()}
    p2["h0"] = run_fwd(p1)["h_final"]
    g2 = run_bwd(p2, dy[:, L1:], dh_final=dhf)
    g1 = run_bwd(p1, dy[:, :L1], dh_final=g2["dh0"])
    for k in ("dx", "ddelta_raw", "dz", "dB", "dC"):
        np.testing.assert_allclose(np.concatenate([g1[k], g2[k]], 1), full[k], rtol=1e-11, atol=1e-12, err_msg=k)
    for k in ("dA_log", "dD", "d_dt_bias"):
        np.testing.assert_allclose(g1[k] + g2[k], full[k], rtol=1e-11, atol=1e-12, err_msg=k)
    np.testing.assert_allclose(g1["dh0"], full["dh0"], rtol=1e-11, atol=1e-12)


def test_zero_final_gradient_is_the_default():
    rng = np.random.default_rng(64)
    p = rand_problem(rng, 2, 9, 3, 4)
    dy = rng.standard_normal((2, 9, 3))
    a = run_bwd(p, dy)
    z = run_bwd(p, dy, dh_final=np.zeros((2, 3, 4)))
    for k in a:
        if a[k] is not None:
            assert np.array_equal(a[k], z[k]), k


# ------------------------------------------------------------- step-size clamp

def _clamp_bounds(p, lo_q=0.3, hi_q=0.7, gap=1e-4):
    """bounds at quantiles of softplus over the problem, nudged so that no step's
    softplus lies within `gap` of a bound (central differences never cross a kink)"""
    sp = softplus_ref(p["delta_raw"] + p["dt_bias"][None, None, :]).ravel()
    lo, hi = np.quantile(sp, lo_q), np.quantile(sp, hi_q)
    for _ in range(100):
        if np.min(np.abs(sp - lo)) > gap and np.min(np.abs(sp - hi)) > gap:
            break
        lo *= 1.0 + 3 * gap
        hi *= 1.0 - 3 * gap
    assert np.min(np.abs(sp - lo)) > gap and np.min(np.abs(sp - hi)) > gap
    assert np.any(sp < lo) and np.any(sp > hi) and np.any((sp > lo) & (sp < hi))
    return float(lo), float(hi)


@pytest.mark.parametrize("gated", [False, True])
def test_clamped_backward_matches_central_differences(gated):
    """Delta = clamp(softplus, dt_min, dt_max) with some steps below, some above and
    some inside the bounds (mamba3_preprocess_backward.slang's dt clamp and mask)."""
    rng = np.random.default_rng(71 if gated else 72)
    b, l, d, n = 2, 6, 3, 2
    p = rand_problem(rng, b, l, d, n, gated=gated, h0=True, dscale=2.0)
    lo, hi = _clamp_bounds(p)
    dy = rng.standard_normal((b, l, d))
    dhf = rng.standard_normal((b, d, n))
    g = run_bwd(p, dy, dh_final=dhf, dt_min=lo, dt_max=hi)

    def loss(q):
        r = run_fwd(q, dt_min=lo, dt_max=hi)
        return float(np.sum(dy * r["y"]) + np.sum(dhf * r["h_final"]))

    names = [k for k in list(GRAD_OF) + ["h0"] if p.get(k) is not None]
    fd = _fd_grads(p, loss, names)
    for name in names:
        gname = GRAD_OF.get(name, "dh0")
        scale = max(1.0, np.abs(fd[name]).max())
        np.testing.assert_allclose(g[gname], fd[name], rtol=1e-6, atol=1e-6 * scale, err_msg=name)
    # the clamped steps pass no gradient to delta_raw
    sp = softplus_ref(p["delta_raw"] + p["dt_bias"][None, None, :])
    assert np.all(g["ddelta_raw"][(sp < lo) | (sp > hi)] == 0.0)


@pytest.mark.parametrize("L", [1, 300])
def test_clamp_to_one_value_gives_the_constant_step_closed_form(L):
    """dt_min = dt_max = c makes Delta = c whatever delta_raw is: with x, B, C, z
    constant in time the scan is the geometric sum with a = exp(c A)."""
    rng = np.random.default_rng(80 + L)
    b, d, n, c = 2, 3, 4, 0.037
    xc = rng.standard_normal((b, d))
    zc = rng.standard_normal((b, d))
    Bc = rng.standard_normal((b, n))
    Cc = rng.standard_normal((b, n))
    A_log = np.log(rng.uniform(0.05, 3.0, (d, n)))
    Dsk = rng.standard_normal(d)
    h0 = rng.standard_normal((b, d, n))
    rep = lambda a: np.repeat(a[:, None, :], L, axis=1)
    raw = 3.0 * rng.standard_normal((b, L, d))  # varies in time; the clamp removes it
    res = oracle.fwd(rep(xc), raw, rep(Bc), rep(Cc), A_log, D=Dsk, dt_bias=rng.standard_normal(d),
                     z=rep(zc), h0=h0, dt_min=c, dt_max=c)
    A = -np.exp(A_log)
    a = np.exp(c * A)[None]                                       # [1, d, n]
    u = c * Bc[:, None, :] * xc[:, :, None]                       # [b, d, n]
    ak = a[:, None] ** np.arange(1, L + 1)[None, :, None, None]   # [b?, L, d, n]
    h = ak * h0[:, None] + u[:, None] * (1 - ak) / (1 - a[:, None])
    s = np.einsum("bldn,bn->bld", h, Cc) + Dsk[None, None, :] * xc[:, None, :]
    y = s * silu_ref(zc)[:, None, :]
    np.testing.assert_allclose(res["y"], y, rtol=1e-11, atol=1e-12 * np.abs(y).max())
    np.testing.assert_allclose(res["h_final"], h[:, -1], rtol=1e-11, atol=1e-12)


def test_clamp_that_never_binds_changes_nothing():
    rng = np.random.default_rng(90)
    p = rand_problem(rng, 2, 40, 5, 3)
    sp = softplus_ref(p["delta_raw"] + p["dt_bias"][None, None, :])
    lo, hi = 0.5 * sp.min(), 2.0 * sp.max()
    dy = rng.standard_normal((2, 40, 5))
    a, c = run_fwd(p), run_fwd(p, dt_min=lo, dt_max=hi)
    assert np.array_equal(a["y"], c["y"]) and np.array_equal(a["h_final"], c["h_final"])
    ga, gc = run_bwd(p, dy), run_bwd(p, dy, dt_min=lo, dt_max=hi)
    for k in ga:
        if ga[k] is not None:
            assert np.array_equal(ga[k], gc[k]), k


def test_clamped_scan_of_length_one_equals_clamped_step():
    rng = np.random.default_rng(91)
    p = rand_problem(rng, 3, 1, 7, 5, dscale=2.0)
    sp = softplus_ref(p["delta_raw"] + p["dt_bias"][None, None, :])
    lo, hi = np.quantile(sp, 0.3), np.quantile(sp, 0.7)
    sc = run_fwd(p, dt_min=lo, dt_max=hi)
    st = oracle.step(p["h0"], p["x"][:, 0], p["delta_raw"][:, 0], p["B"][:, 0], p["C"][:, 0], p["A_log"],
                     D=p["D"], dt_bias=p["dt_bias"], z=p["z"][:, 0], dt_min=lo, dt_max=hi)
    np.testing.assert_allclose(st["y"], sc["y"][:, 0], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(st["state"], sc["h_final"], rtol=1e-15, atol=1e-15)


def test_invalid_clamp_bounds_are_rejected():
    rng = np.random.default_rng(92)
    p = rand_problem(rng, 1, 3, 2, 2)
    for lo, hi in ((0.2, 0.1), (-0.1, 1.0), (float("nan"), 1.0)):
        with pytest.raises(RuntimeError):
            run_fwd(p, dt_min=lo, dt_max=hi)
