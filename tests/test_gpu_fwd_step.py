"""GPU parity of the forward scan and the decode step against the fp64 oracle.

The HIP path is called through the C ABI (selective_state_space_03_amd.ops); the
oracle runs on the same seeded inputs.  Bounds: max relative error (RMS floor)
1e-4 for fp32 I/O and 2e-2 for bf16 I/O.  Small cases span several channel
tiles, several time tiles and ragged tails; the named full-size workloads are
checked on sampled channels (channels are independent, so the oracle runs on
exactly those channels).  Invariants: L=1 scan equals the step, zero input gives
exactly zero, segment composition through h0/h_final, bit-identical repeats.
"""
import os

import numpy as np
import pytest

import oracle
from _helpers import host, rel_err, say, to_dev, to_dev32, tol
from selective_state_space_03_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from selective_state_space_03_amd import ops
    ops.lib()  # the HIP library must load; its absence is a failure, never a fallback


def ops():
    from selective_state_space_03_amd import ops as o
    return o


def gpu_fwd(inp, h_final=True):
    io = inp["io"]
    y, hf = ops().ssm_scan_fwd(to_dev(inp["x"], io), to_dev(inp["delta_raw"], io), to_dev(inp["B"], io),
                               to_dev(inp["C"], io), to_dev32(inp["A_log"]), D_skip=to_dev32(inp["D"]),
                               dt_bias=to_dev32(inp["dt_bias"]), z=to_dev(inp["z"], io),
                               h0=to_dev32(inp.get("h0")), return_final_state=h_final)
    torch.cuda.synchronize()
    return host(y), (host(hf) if hf is not None else None)


def oracle_fwd(inp, chans=None):
    sel = (lambda a: a) if chans is None else (lambda a: a[..., chans])
    selp = (lambda a: a) if chans is None else (lambda a: a[chans])
    h0 = inp.get("h0")
    return oracle.fwd(sel(inp["x"]), sel(inp["delta_raw"]), inp["B"], inp["C"], selp(inp["A_log"]),
                      D=selp(inp["D"]), dt_bias=selp(inp["dt_bias"]),
                      z=None if inp["z"] is None else sel(inp["z"]),
                      h0=None if h0 is None else (h0 if chans is None else h0[:, chans]))


SMALL_FWD = [
    # name, workload, overrides
    ("fwd_small_exact", "fwd_small", {}),
    ("ragged_gated_h0", "fwd_b8_l2048_d1536", dict(batch=2, seqlen=37, dim=100, random_h0=True)),
    ("tiles_and_tail", "fwd_b8_l2048_d1536", dict(batch=3, seqlen=300, dim=130)),
    ("n8", "fwd_b8_l2048_d1536", dict(batch=2, seqlen=75, dim=64, dstate=8)),
    ("n5_masked_states", "fwd_b8_l2048_d1536", dict(batch=2, seqlen=129, dim=70, dstate=5, random_h0=True)),
    ("n12", "fwd_b8_l2048_d1536", dict(batch=1, seqlen=50, dim=200, dstate=12)),
    ("n1", "fwd_small", dict(batch=2, seqlen=40, dim=3, dstate=1)),
    ("single_element", "fwd_small", dict(batch=1, seqlen=1, dim=1, dstate=16)),
    ("ungated_long", "fwd_small", dict(batch=1, seqlen=5000, dim=65, dstate=16)),
    ("bf16_gated", "fwd_bf16_b4_l4096_d4096", dict(batch=2, seqlen=200, dim=192, random_h0=True)),
    ("bf16_ragged_n7", "fwd_bf16_b4_l4096_d4096", dict(batch=3, seqlen=33, dim=77, dstate=7)),
]


@pytest.mark.parametrize("name,wl,over", SMALL_FWD, ids=[c[0] for c in SMALL_FWD])
def test_fwd_parity_small(name, wl, over):
    w = W.WORKLOADS[wl]
    inp = W.make_inputs(w, **over)
    say("fwd %s B=%d L=%d D=%d N=%d io=%s gated=%s" % (name, inp["batch"], inp["seqlen"], inp["dim"],
                                                        inp["dstate"], inp["io"], inp["z"] is not None))
    y, hf = gpu_fwd(inp)
    ref = oracle_fwd(inp)
    assert rel_err(y, ref["y"]) <= tol(inp["io"]), rel_err(y, ref["y"])
    assert rel_err(hf, ref["h_final"]) <= tol(inp["io"]), rel_err(hf, ref["h_final"])


@pytest.mark.parametrize("wl", ["fwd_b8_l2048_d1536", "fwd_bf16_b4_l4096_d4096", "fwdbwd_b4_l2048_d2048"])
def test_fwd_parity_full_size_sampled_channels(wl):
    """Full-size workload as the benchmark runs it; the oracle computes sampled
    channels (first/last of the tensor, tile edges, random) over the whole sequence."""
    w = W.WORKLOADS[wl]
    inp = W.make_inputs(w, with_dy=False)
    say("fwd full %s" % wl)
    y, hf = gpu_fwd(inp)
    rng = np.random.default_rng(5)
    d = inp["dim"]
    chans = sorted(set([0, 1, 63, 64, 65, d // 2, d - 65, d - 64, d - 1] + list(rng.integers(0, d, 15))))
    ref = oracle_fwd(inp, chans)
    assert rel_err(y[..., chans], ref["y"]) <= tol(inp["io"])
    assert rel_err(hf[:, chans], ref["h_final"]) <= tol(inp["io"])


def test_fwd_zero_input_gives_exact_zero():
    inp = W.make_inputs(W.WORKLOADS["fwd_b8_l2048_d1536"], batch=2, seqlen=100, dim=96)
    inp["x"] = np.zeros_like(inp["x"])
    say("fwd zero input")
    y, hf = gpu_fwd(inp)
    assert np.all(y == 0) and np.all(hf == 0)


def test_fwd_composition_through_final_state():
    inp = W.make_inputs(W.WORKLOADS["fwd_b8_l2048_d1536"], batch=2, seqlen=250, dim=128, random_h0=True)
    L1 = 97
    say("fwd composition")
    y, hf = gpu_fwd(inp)
    a = {k: (v[:, :L1] if k in ("x", "delta_raw", "z", "B", "C") else v) for k, v in inp.items()}
    ya, hfa = gpu_fwd(a)
    b = {k: (v[:, L1:] if k in ("x", "delta_raw", "z", "B", "C") else v) for k, v in inp.items()}
    b["h0"] = hfa
    yb, hfb = gpu_fwd(b)
    assert rel_err(np.concatenate([ya, yb], 1), y) <= 1e-5
    assert rel_err(hfb, hf) <= 1e-5


def test_fwd_is_bit_identical_across_runs():
    inp = W.make_inputs(W.WORKLOADS["fwd_b8_l2048_d1536"], batch=2, seqlen=513, dim=200, random_h0=True)
    say("fwd determinism")
    runs = [gpu_fwd(inp) for _ in range(3)]
    for y, hf in runs[1:]:
        assert np.array_equal(y, runs[0][0]) and np.array_equal(hf, runs[0][1])


# ------------------------------------------------------------------ step

def gpu_step(inp):
    io = inp["io"]
    st = to_dev32(inp["state"])
    y = ops().ssm_scan_step(st, to_dev(inp["x"], io), to_dev(inp["delta_raw"], io), to_dev(inp["B"], io),
                            to_dev(inp["C"], io), to_dev32(inp["A_log"]), D_skip=to_dev32(inp["D"]),
                            dt_bias=to_dev32(inp["dt_bias"]), z=to_dev(inp["z"], io))
    torch.cuda.synchronize()
    return host(y), host(st)


def oracle_step(inp):
    return oracle.step(inp["state"], inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"],
                       D=inp["D"], dt_bias=inp["dt_bias"], z=inp["z"])


STEP_CASES = [
    ("decode_full_b256_d5120", {}),
    ("ragged", dict(batch=3, dim=77)),
    ("n4_one_lane_per_pair", dict(batch=5, dim=130, dstate=4)),
    ("n8_two_lanes_per_pair", dict(batch=5, dim=130, dstate=8)),
    ("n5_scalar_path", dict(batch=4, dim=65, dstate=5)),
    ("n13_scalar_path", dict(batch=2, dim=33, dstate=13)),
    ("ungated", dict(batch=4, dim=100, gated=False)),
    ("single", dict(batch=1, dim=1, dstate=1)),
]


@pytest.mark.parametrize("name,over", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_step_parity(name, over):
    inp = W.make_inputs(W.WORKLOADS["step_b256_d5120"], **over)
    say("step %s B=%d D=%d N=%d" % (name, inp["batch"], inp["dim"], inp["dstate"]))
    y, st = gpu_step(inp)
    ref = oracle_step(inp)
    assert rel_err(y, ref["y"]) <= 1e-4
    assert rel_err(st, ref["state"]) <= 1e-4


def test_step_bf16():
    w = W.Workload("step_bf16", "step", 64, 1, 300, 16, "bf16", True, "mamba", 77)
    inp = W.make_inputs(w)
    say("step bf16")
    y, st = gpu_step(inp)
    ref = oracle_step(inp)
    assert rel_err(y, ref["y"]) <= 2e-2
    assert rel_err(st, ref["state"]) <= 1e-4  # the state is fp32


def test_scan_of_length_one_equals_step():
    inp = W.make_inputs(W.WORKLOADS["fwd_b8_l2048_d1536"], batch=4, seqlen=1, dim=200, random_h0=True)
    say("L=1 scan vs step")
    y, hf = gpu_fwd(inp)
    st_inp = dict(inp)
    st_inp.update(state=inp["h0"], x=inp["x"][:, 0], delta_raw=inp["delta_raw"][:, 0], z=inp["z"][:, 0],
                  B=inp["B"][:, 0], C=inp["C"][:, 0])
    ys, sts = gpu_step(st_inp)
    assert rel_err(ys, y[:, 0]) <= 1e-5
    assert rel_err(sts, hf) <= 1e-5


def test_step_is_bit_identical_across_runs():
    inp = W.make_inputs(W.WORKLOADS["step_b256_d5120"], batch=16, dim=1000)
    say("step determinism")
    runs = [gpu_step(inp) for _ in range(3)]
    for y, st in runs[1:]:
        assert np.array_equal(y, runs[0][0]) and np.array_equal(st, runs[0][1])
