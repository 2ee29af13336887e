"""GPU checks of the fused decode step (include/ssm_decode.h): the depthwise conv1d step
and the selective-scan step for one token, in one launch.

* Bit for bit against the same tokens through ssm_conv1d_step and then ssm_scan_step_ex
  (the convolution's output fed to the scan as x), over three tokens in a row with both
  states carried.  The cases cover fp32 and bf16 I/O, gated and ungated, with and without
  SiLU, widths 1, 2, 4 and 8, and d_state 4, 8 and 16 (one, two and four lanes per
  channel). They also cover a d_state of 5 (the scalar path), ragged channel counts,
  with and without the u output, the step-size clamp, and the decode workload's full
  size (256 x 5120, d_state 16, width 4).
* Against the oracle: the oracle's conv step and then its scan step, at the documented
  tolerances (1e-4 for fp32 I/O, 2e-2 for bf16 I/O with an fp32 state).
"""
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
    ops.lib()


def make_case(batch, dim, dstate, width, io="f32", gated=True, silu=True, bias=True, seed=0):
    """Scan-step inputs (state, A_log, D, dt_bias) and conv-step inputs (state, weight,
    bias) of the workloads' distributions, plus three tokens (x before the convolution,
    delta_raw, B, C, z), all rounded to io."""
    w = W.Workload("decode", "step", batch, 1, dim, dstate, io, gated, "mamba", 4400 + seed)
    sc = W.make_inputs(w)
    cv = W.make_conv_inputs(W.CONV_WORKLOADS["conv_step_b256_d5120_k4"], batch=batch, dim=dim, width=width,
                            silu=silu, io=io, seed=4500 + seed)
    rng = np.random.default_rng(4600 + seed)
    toks = []
    for _ in range(3):
        toks.append({k: W.round_to_io(rng.standard_normal(shp), io) for k, shp in
                     (("x", (batch, dim)), ("delta_raw", (batch, dim)), ("B", (batch, dstate)),
                      ("C", (batch, dstate)), ("z", (batch, dim)))})
        toks[-1]["delta_raw"] = toks[-1]["delta_raw"] - 1.0 if io == "f32" else toks[-1]["delta_raw"]
        if not gated:
            toks[-1]["z"] = None
    return dict(io=io, width=width, silu=silu, state=sc["state"], A_log=sc["A_log"], D=sc["D"],
                dt_bias=sc["dt_bias"], conv_state=cv["state"], weight=cv["weight"],
                bias=cv["bias"] if bias else None, toks=toks)


def run_pair(c, dt_min=None, dt_max=None):
    """the two separate calls, token by token; returns per-token (y, u) and the final states"""
    from selective_state_space_03_amd import ops
    io, k = c["io"], c["width"]
    cs = to_dev(c["conv_state"], io) if k > 1 else None
    st = to_dev32(c["state"])
    w, b = to_dev32(c["weight"]), to_dev32(c["bias"])
    A, D, dtb = to_dev32(c["A_log"]), to_dev32(c["D"]), to_dev32(c["dt_bias"])
    outs = []
    for t in c["toks"]:
        u = ops.conv1d_step(cs, to_dev(t["x"], io), w, bias=b, silu=c["silu"])
        y = ops.ssm_scan_step(st, u, to_dev(t["delta_raw"], io), to_dev(t["B"], io), to_dev(t["C"], io), A,
                              D_skip=D, dt_bias=dtb, z=to_dev(t["z"], io), dt_min=dt_min, dt_max=dt_max)
        outs.append((host(y), host(u)))
    torch.cuda.synchronize()
    return outs, (host(cs) if k > 1 else None), host(st)


def run_fused(c, want_u=True, dt_min=None, dt_max=None):
    from selective_state_space_03_amd import ops
    io, k = c["io"], c["width"]
    cs = to_dev(c["conv_state"], io) if k > 1 else None
    st = to_dev32(c["state"])
    w, b = to_dev32(c["weight"]), to_dev32(c["bias"])
    A, D, dtb = to_dev32(c["A_log"]), to_dev32(c["D"]), to_dev32(c["dt_bias"])
    outs = []
    for t in c["toks"]:
        x = to_dev(t["x"], io)
        u = torch.empty_like(x) if want_u else None
        y = ops.decode_step(cs, x, w, st, to_dev(t["delta_raw"], io), to_dev(t["B"], io), to_dev(t["C"], io), A,
                            conv_bias=b, silu=c["silu"], D_skip=D, dt_bias=dtb, z=to_dev(t["z"], io), u=u,
                            dt_min=dt_min, dt_max=dt_max)
        outs.append((host(y), host(u) if want_u else None))
    torch.cuda.synchronize()
    return outs, (host(cs) if k > 1 else None), host(st)


CASES = [
    # (name, batch, dim, dstate, width, io, gated, silu, bias)
    ("n16_k4", 8, 300, 16, 4, "f32", True, True, True),
    ("n8_k2_ungated", 5, 130, 8, 2, "f32", False, True, True),
    ("n4_k8_no_silu", 3, 77, 4, 8, "f32", True, False, False),
    ("n5_scalar_k4", 4, 65, 5, 4, "f32", True, True, True),
    ("width1", 2, 70, 16, 1, "f32", True, True, True),
    ("bf16_n16_k4", 4, 130, 16, 4, "bf16", True, True, True),
    ("bf16_n8_k3_ungated", 3, 99, 8, 3, "bf16", False, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_step_equals_the_two_calls_bit_for_bit(case):
    name, b, d, n, k, io, gated, silu, bias = case
    say("decode step %s B=%d D=%d N=%d K=%d io=%s" % (name, b, d, n, k, io))
    c = make_case(b, d, n, k, io, gated, silu, bias, seed=len(name))
    ref, cs_ref, st_ref = run_pair(c)
    for want_u in (True, False):
        got, cs, st = run_fused(c, want_u=want_u)
        for i, ((y, u), (yr, ur)) in enumerate(zip(got, ref)):
            assert np.array_equal(y, yr), (name, i)
            if want_u:
                assert np.array_equal(u, ur), (name, i)
        if k > 1:
            assert np.array_equal(cs, cs_ref), name
        assert np.array_equal(st, st_ref), name


def test_decode_step_with_the_step_size_clamp():
    say("decode step with the step-size clamp")
    c = make_case(4, 100, 16, 4, seed=3)
    ref, cs_ref, st_ref = run_pair(c, dt_min=0.05, dt_max=0.2)
    got, cs, st = run_fused(c, dt_min=0.05, dt_max=0.2)
    for (y, u), (yr, ur) in zip(got, ref):
        assert np.array_equal(y, yr) and np.array_equal(u, ur)
    assert np.array_equal(cs, cs_ref) and np.array_equal(st, st_ref)


def test_decode_step_full_size_equals_the_two_calls():
    say("decode step 256 x 5120, d_state 16, width 4")
    c = make_case(256, 5120, 16, 4, seed=9)
    c["toks"] = c["toks"][:1]
    ref, cs_ref, st_ref = run_pair(c)
    got, cs, st = run_fused(c)
    assert np.array_equal(got[0][0], ref[0][0]) and np.array_equal(got[0][1], ref[0][1])
    assert np.array_equal(cs, cs_ref) and np.array_equal(st, st_ref)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_step_matches_the_oracle(io):
    say("decode step vs oracle, io=%s" % io)
    c = make_case(6, 200, 16, 4, io=io, seed=11)
    got, cs, st = run_fused(c)
    cs_o, st_o = c["conv_state"].astype(np.float64), c["state"].astype(np.float64)
    for i, t in enumerate(c["toks"]):
        cr = oracle.conv_step(cs_o, t["x"], c["weight"], c["bias"], silu=c["silu"])
        cs_o = cr["state"]
        sr = oracle.step(st_o, cr["out"], t["delta_raw"], t["B"], t["C"], c["A_log"], D=c["D"],
                         dt_bias=c["dt_bias"], z=t["z"])
        st_o = sr["state"]
        assert rel_err(got[i][0], sr["y"]) <= tol(io), i
        assert rel_err(got[i][1], cr["out"]) <= tol(io), i
    assert np.array_equal(cs, cs_o.astype(np.float32))  # shifted copies of the inputs: exact
    assert rel_err(st, st_o) <= (1e-4 if io == "f32" else 2e-2)
