"""Pins of the SSD chunk-cumsum oracle against facts that do not come from it.

* constant dt: dA_cumsum[l] = (l + 1) * g(dt + bias) * A inside every chunk, with the
  ragged last chunk padded by zeros (closed form);
* chunk composition: the last entry of every chunk equals A times the total of that
  chunk's dt_out computed on its own, and the chunk width does not change the
  per-position dt_out;
* backward: central differences of L = sum(ddA * dA_cumsum) + sum(ddt_out * dt_out)
  with respect to every dt, A and dt_bias element, with softplus on and off and with
  a binding clamp (inputs kept away from the clamp's kinks);
* clamped positions pass no gradient to dt; the (b, chunk) partials add to dA and
  d_dt_bias.
"""
import numpy as np
import pytest

from oracle import ssd_cumsum_oracle as S


def test_constant_dt_closed_form():
    b, L, H, W = 2, 37, 3, 8
    dt = np.full((b, L, H), -0.7)
    A = np.array([-0.5, -1.0, -2.0])
    bias = np.array([0.1, 0.2, 0.3])
    cs, dto = S.chunk_cumsum_fwd(dt, A, bias, W, dt_softplus=True)
    sp = np.log1p(np.exp(-0.7 + bias))
    nc = (L + W - 1) // W
    for c in range(nc):
        n_valid = min(W, L - c * W)
        for l in range(W):
            k = min(l + 1, n_valid)
            np.testing.assert_allclose(cs[:, :, c, l], np.broadcast_to(k * sp * A, (b, H)), rtol=1e-14)
            want = sp if l < n_valid else np.zeros(H)
            np.testing.assert_allclose(dto[:, :, c, l], np.broadcast_to(want, (b, H)), rtol=1e-15)


def test_chunk_totals_and_width_independence():
    rng = np.random.default_rng(5)
    b, L, H = 2, 50, 4
    dt = rng.standard_normal((b, L, H))
    A = -rng.uniform(0.1, 2.0, H)
    bias = rng.standard_normal(H) * 0.3
    cs8, dto8 = S.chunk_cumsum_fwd(dt, A, bias, 8, dt_min=0.2, dt_max=1.5)
    cs16, dto16 = S.chunk_cumsum_fwd(dt, A, bias, 16, dt_min=0.2, dt_max=1.5)
    flat8 = dto8.reshape(b, H, -1)[:, :, :L]
    flat16 = dto16.reshape(b, H, -1)[:, :, :L]
    assert np.array_equal(flat8, flat16)
    for c in range(cs8.shape[2]):
        tot = np.sum(dto8[:, :, c, :], axis=2) * A[None, :]
        np.testing.assert_allclose(cs8[:, :, c, -1], tot, rtol=1e-13, atol=1e-15)


def _loss(dt, A, bias, ddA, ddt_out, W, sp, lo, hi):
    cs, dto = S.chunk_cumsum_fwd(dt, A, bias, W, sp, lo, hi)
    return float(np.sum(ddA * cs) + np.sum(ddt_out * dto))


@pytest.mark.parametrize("softplus,clamp", [(True, False), (True, True), (False, True)])
def test_backward_matches_central_differences(softplus, clamp):
    rng = np.random.default_rng(11 + 2 * softplus + clamp)
    b, L, H, W = 2, 13, 3, 4
    dt = rng.standard_normal((b, L, H)) * (1.0 if softplus else 0.5) + (0.0 if softplus else 1.0)
    A = -rng.uniform(0.2, 2.0, H)
    bias = rng.standard_normal(H) * 0.3
    nc = (L + W - 1) // W
    ddA = rng.standard_normal((b, H, nc, W))
    ddt_out = rng.standard_normal((b, H, nc, W))
    lo, hi = 0.0, float("inf")
    if clamp:
        pre = S._g(dt + bias[None, None, :], softplus).ravel()
        lo, hi = np.quantile(pre, 0.25), np.quantile(pre, 0.75)
        for _ in range(1000):  # keep every element clear of the kinks
            if min(np.min(np.abs(pre - lo)), np.min(np.abs(pre - hi))) > 1e-3:
                break
            lo, hi = lo * 1.002 + 1e-4, hi * 0.998 - 1e-4
        assert min(np.min(np.abs(pre - lo)), np.min(np.abs(pre - hi))) > 1e-3
        assert np.any(pre < lo) and np.any(pre > hi)
    r = S.chunk_cumsum_bwd(ddA, ddt_out, dt, A, bias, W, softplus, lo, hi)
    for name, arr, key in (("dt", dt, "ddt"), ("A", A, "dA"), ("bias", bias, "d_dt_bias")):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            h = 1e-6 * max(1.0, abs(arr[idx]))
            args = {"dt": dt, "A": A, "bias": bias}
            up, dn = arr.copy(), arr.copy()
            up[idx] += h
            dn[idx] -= h
            args[name] = up
            lp = _loss(args["dt"], args["A"], args["bias"], ddA, ddt_out, W, softplus, lo, hi)
            args[name] = dn
            lm = _loss(args["dt"], args["A"], args["bias"], ddA, ddt_out, W, softplus, lo, hi)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(r[key], fd, rtol=1e-6, atol=1e-7 * max(1.0, np.abs(fd).max()), err_msg=name)
    if clamp:
        pre = S._g(dt + bias[None, None, :], softplus)
        assert np.all(r["ddt"][(pre < lo) | (pre > hi)] == 0.0)
    np.testing.assert_allclose(r["dA"], r["dA_partial"].sum(axis=(0, 1)), rtol=1e-13)
    np.testing.assert_allclose(r["d_dt_bias"], r["db_partial"].sum(axis=(0, 1)), rtol=1e-13)
