"""Pins of the fp64 conv1d oracle (CPU only) to things it does not compute itself.

Pins (definitions in oracle/conv1d_oracle.c):
  * numpy.convolve (a library routine) gives the pre-activation of every channel;
  * a width-1 filter is an elementwise affine map followed by SiLU (closed form);
  * a unit impulse reproduces the taps in reverse order (closed form);
  * stepping the decode function through a sequence from a zero state reproduces the
    sequence forward (separate code paths);
  * the backward matches fp64 central differences of the loss sum(dout * out) for
    every input, weight and bias element, with and without SiLU;
  * with zero weights, dx = 0 and dbias = sum of dout * silu'(bias).
"""
import numpy as np
import pytest

import oracle
from selective_state_space_03_amd import workloads as W


def np_silu(z):
    return z / (1.0 + np.exp(-z))


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("k", [1, 2, 4, 7])
def test_matches_numpy_convolve(silu, k):
    inp = W.make_conv_inputs(W.CONV_WORKLOADS["conv_small"], batch=2, seqlen=29, dim=5, width=k)
    x, w, bias = inp["x"].astype(np.float64), inp["weight"].astype(np.float64), inp["bias"].astype(np.float64)
    out = oracle.conv_fwd(x, w, bias, silu=silu)
    b, l, d = x.shape
    for bb in range(b):
        for dd in range(d):
            p = np.convolve(x[bb, :, dd], w[dd, ::-1])[:l] + bias[dd]
            want = np_silu(p) if silu else p
            np.testing.assert_allclose(out[bb, :, dd], want, rtol=1e-13, atol=1e-13)


def test_width_one_is_elementwise():
    inp = W.make_conv_inputs(W.CONV_WORKLOADS["conv_small"], batch=2, seqlen=11, dim=6, width=1)
    x, w, bias = inp["x"].astype(np.float64), inp["weight"].astype(np.float64), inp["bias"].astype(np.float64)
    out = oracle.conv_fwd(x, w, bias, silu=True)
    np.testing.assert_allclose(out, np_silu(x * w[:, 0] + bias), rtol=1e-14, atol=1e-15)


def test_impulse_reproduces_taps_in_reverse():
    k, l, t0 = 4, 12, 5
    w = np.array([[0.5, -1.25, 2.0, 3.5]])
    x = np.zeros((1, l, 1))
    x[0, t0, 0] = 1.0
    out = oracle.conv_fwd(x, w, np.zeros(1), silu=False)[0, :, 0]
    want = np.zeros(l)
    for j in range(k):  # out[t0 + j] sees the impulse at tap K-1-j
        want[t0 + j] = w[0, k - 1 - j]
    np.testing.assert_array_equal(out, want)


@pytest.mark.parametrize("k", [1, 3, 4])
def test_steps_reproduce_the_sequence_forward(k):
    inp = W.make_conv_inputs(W.CONV_WORKLOADS["conv_small"], batch=3, seqlen=17, dim=4, width=k)
    x, w, bias = inp["x"].astype(np.float64), inp["weight"].astype(np.float64), inp["bias"].astype(np.float64)
    seq = oracle.conv_fwd(x, w, bias, silu=True)
    b, l, d = x.shape
    state = np.zeros((b, d, k - 1))
    for t in range(l):
        r = oracle.conv_step(state, x[:, t], w, bias, silu=True)
        state = r["state"]
        np.testing.assert_allclose(r["out"], seq[:, t], rtol=1e-14, atol=1e-15)
    if k > 1:  # the state holds the last K-1 inputs, oldest first
        np.testing.assert_array_equal(state, np.transpose(x[:, l - (k - 1):], (0, 2, 1)))


@pytest.mark.parametrize("silu", [False, True])
def test_backward_matches_central_differences(silu):
    inp = W.make_conv_inputs(W.CONV_WORKLOADS["conv_small"], batch=2, seqlen=6, dim=3, width=3)
    x, w, bias = inp["x"].astype(np.float64), inp["weight"].astype(np.float64), inp["bias"].astype(np.float64)
    dout = inp["dout"].astype(np.float64)
    g = oracle.conv_bwd(x, w, dout, bias, silu=silu)

    def loss(xx, ww, bb):
        return float(np.sum(dout * oracle.conv_fwd(xx, ww, bb, silu=silu)))

    for name, arr in (("dx", x), ("dw", w), ("dbias", bias)):
        num = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            h = 1e-6 * max(1.0, abs(arr[idx]))
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = [ap if a is arr else a for a in (x, w, bias)]
            args_m = [am if a is arr else a for a in (x, w, bias)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_zero_weights_backward():
    inp = W.make_conv_inputs(W.CONV_WORKLOADS["conv_small"], batch=2, seqlen=9, dim=4, width=4)
    x, bias, dout = inp["x"].astype(np.float64), inp["bias"].astype(np.float64), inp["dout"].astype(np.float64)
    g = oracle.conv_bwd(x, np.zeros((4, 4)), dout, bias, silu=True)
    sg = 1.0 / (1.0 + np.exp(-bias))
    dsilu = sg * (1.0 + bias * (1.0 - sg))
    assert np.all(g["dx"] == 0.0)
    np.testing.assert_allclose(g["dbias"], dout.sum(axis=(0, 1)) * dsilu, rtol=1e-13)
