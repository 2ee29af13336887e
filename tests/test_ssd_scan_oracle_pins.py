"""Pins of the SSD scan oracle against facts that do not come from it.

* reduction to the Mamba selective scan: an SSD head with headdim P is P channels of
  the selective scan whose decay rate A[d, n] is the head's A for every state, whose
  step is the head's dt (passed as softplus^-1(dt) with no bias), and whose B, C are
  shared -- so the independently written and pinned C oracle of the selective scan
  must give the same y and final state;
* constant inputs: the closed-form geometric sum;
* brute-force unrolling (products of decays) for L <= 6, with an initial state;
* composition of two segments through h0 / h_final; zero input gives zero output;
* backward: fp64 central differences of sum(dy * y) + sum(dh_final * h_final) with
  respect to every element of x, dt, A, B, C, D and h0.
"""
import numpy as np

import oracle
from oracle import ssd_scan_oracle as S


def _inputs(rng, b, L, H, P, N, h0=True):
    x = rng.standard_normal((b, L, H, P))
    dt = rng.uniform(0.01, 0.5, (b, L, H))
    A = -rng.uniform(0.5, 4.0, H)
    Bm = rng.standard_normal((b, L, N))
    Cm = rng.standard_normal((b, L, N))
    D = rng.standard_normal(H)
    hz = rng.standard_normal((b, H, P, N)) if h0 else None
    return x, dt, A, Bm, Cm, D, hz


def test_reduces_to_the_selective_scan_oracle():
    rng = np.random.default_rng(11)
    b, L, H, P, N = 2, 13, 2, 3, 4
    x, dt, A, Bm, Cm, D, h0 = _inputs(rng, b, L, H, P, N)
    got = S.ssd_scan_fwd(x, dt, A, Bm, Cm, D, h0)
    Dm = H * P
    xf = x.reshape(b, L, Dm)
    raw = np.repeat(np.log(np.expm1(dt)), P, axis=2)        # softplus(raw) = dt
    A_log = np.repeat(np.log(-A), P)[:, None] * np.ones((1, N))
    ref = oracle.fwd(xf, raw, Bm, Cm, A_log, D=np.repeat(D, P), h0=h0.reshape(b, Dm, N), nthreads=1)
    np.testing.assert_allclose(got["y"].reshape(b, L, Dm), ref["y"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["h_final"].reshape(b, Dm, N), ref["h_final"], rtol=1e-10, atol=1e-12)


def test_constant_inputs_closed_form():
    b, L, H, P, N = 1, 300, 2, 3, 5
    rng = np.random.default_rng(3)
    xv, Bv, Cv = rng.standard_normal((H, P)), rng.standard_normal(N), rng.standard_normal(N)
    dt0 = np.array([0.05, 0.2])
    A = np.array([-1.0, -3.0])
    D = np.array([0.5, -2.0])
    x = np.broadcast_to(xv, (b, L, H, P))
    dt = np.broadcast_to(dt0, (b, L, H))
    out = S.ssd_scan_fwd(x, dt, A, np.broadcast_to(Bv, (b, L, N)), np.broadcast_to(Cv, (b, L, N)), D)
    for h in range(H):
        a = np.exp(dt0[h] * A[h])
        u = dt0[h] * np.outer(xv[h], Bv)
        for t in (0, 1, 7, L - 1):
            st = u * (1 - a ** (t + 1)) / (1 - a)
            np.testing.assert_allclose(out["y"][0, t, h], st @ Cv + D[h] * xv[h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(out["h_final"][0, h], u * (1 - a ** L) / (1 - a), rtol=1e-12)


def test_bruteforce_unroll():
    rng = np.random.default_rng(7)
    b, L, H, P, N = 1, 6, 2, 2, 3
    x, dt, A, Bm, Cm, D, h0 = _inputs(rng, b, L, H, P, N)
    out = S.ssd_scan_fwd(x, dt, A, Bm, Cm, D, h0)
    for h in range(H):
        for t in range(L):
            decay = lambda s0, s1: np.prod([np.exp(dt[0, r, h] * A[h]) for r in range(s0, s1 + 1)])  # noqa: E731
            st = decay(0, t) * h0[0, h]
            for s in range(t + 1):
                st = st + (decay(s + 1, t) if s < t else 1.0) * dt[0, s, h] * np.outer(x[0, s, h], Bm[0, s])
            np.testing.assert_allclose(out["y"][0, t, h], st @ Cm[0, t] + D[h] * x[0, t, h], rtol=1e-12, atol=1e-13)


def test_segments_compose_and_zero_input():
    rng = np.random.default_rng(9)
    b, L, H, P, N = 2, 40, 2, 4, 3
    x, dt, A, Bm, Cm, D, h0 = _inputs(rng, b, L, H, P, N)
    whole = S.ssd_scan_fwd(x, dt, A, Bm, Cm, D, h0)
    k = 17
    first = S.ssd_scan_fwd(x[:, :k], dt[:, :k], A, Bm[:, :k], Cm[:, :k], D, h0)
    second = S.ssd_scan_fwd(x[:, k:], dt[:, k:], A, Bm[:, k:], Cm[:, k:], D, first["h_final"])
    np.testing.assert_allclose(np.concatenate([first["y"], second["y"]], axis=1), whole["y"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(second["h_final"], whole["h_final"], rtol=1e-12, atol=1e-13)
    zero = S.ssd_scan_fwd(np.zeros_like(x), dt, A, Bm, Cm, D)
    assert np.all(zero["y"] == 0) and np.all(zero["h_final"] == 0)


def test_backward_matches_central_differences():
    rng = np.random.default_rng(21)
    b, L, H, P, N = 1, 5, 2, 2, 3
    x, dt, A, Bm, Cm, D, h0 = _inputs(rng, b, L, H, P, N)
    dy = rng.standard_normal((b, L, H, P))
    dhf = rng.standard_normal((b, H, P, N))
    args = {"x": x, "dt": dt, "A": A, "B": Bm, "C": Cm, "D": D, "h0": h0}

    def loss(a):
        o = S.ssd_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["h0"])
        return float(np.sum(o["y"] * dy) + np.sum(o["h_final"] * dhf))

    g = S.ssd_scan_bwd(x, dt, A, Bm, Cm, dy, D, h0, dhf)
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}
    for k, gk in names.items():
        num = np.zeros_like(args[k])
        for idx in np.ndindex(args[k].shape):
            eps = 1e-6 * max(1.0, abs(args[k][idx]))
            up = {kk: (v.copy() if kk == k else v) for kk, v in args.items()}
            dn = {kk: (v.copy() if kk == k else v) for kk, v in args.items()}
            up[k][idx] += eps
            dn[k][idx] -= eps
            num[idx] = (loss(up) - loss(dn)) / (2 * eps)
        np.testing.assert_allclose(g[gk], num, rtol=1e-6, atol=1e-8, err_msg=k)
