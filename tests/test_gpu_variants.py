"""GPU parity of the variants of the same path against the fp64 oracle.

* Step-size clamp: Delta = clamp(softplus, dt_min, dt_max), with the delta_raw
  gradient masked to steps inside the bounds (forward in every layout and dtype, the
  decode step, the backward).  The bounds sit at quantiles of the inputs' softplus
  values and are moved until no element lies within a relative 1e-5 of a bound: the
  clamp decision is a comparison, and this keeps the fp32 (GPU) and fp64 (oracle)
  decisions identical for every element.
* Sequences carried across segments: dh_final (gradient reaching h_final) in, dh0
  (gradient of h0) out, on shapes with many time segments in the backward; and the
  GPU backward split in two (dh0 of the second part as dh_final of the first)
  against the GPU backward of the whole sequence.
Bounds as elsewhere: max relative error (RMS floor) 1e-4 for fp32, 2e-2 for bf16.
"""
import numpy as np
import pytest

import oracle
from _helpers import host, rel_err, say, to_dev, to_dev32, tol
from selective_state_space_03_amd import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GRADS = ("dx", "ddelta_raw", "dz", "dB", "dC", "dA_log", "dD", "d_dt_bias", "dh0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from selective_state_space_03_amd import ops
    ops.lib()


def ops():
    from selective_state_space_03_amd import ops as o
    return o


def clamp_bounds(inp, lo_q=0.25, hi_q=0.75, gap=1e-5):
    r = inp["delta_raw"].astype(np.float64) + inp["dt_bias"].astype(np.float64)
    sp = np.logaddexp(0.0, r).ravel()
    lo, hi = float(np.quantile(sp, lo_q)), float(np.quantile(sp, hi_q))
    for _ in range(1000):
        ok_lo = np.min(np.abs(sp - lo)) > gap * lo
        ok_hi = np.min(np.abs(sp - hi)) > gap * hi
        if ok_lo and ok_hi:
            break
        lo = lo if ok_lo else lo * (1.0 + 2 * gap)
        hi = hi if ok_hi else hi * (1.0 - 2 * gap)
    assert np.min(np.abs(sp - lo)) > gap * lo and np.min(np.abs(sp - hi)) > gap * hi
    # float32 bounds as the library receives them, and still clear of every element
    lo32, hi32 = float(np.float32(lo)), float(np.float32(hi))
    assert np.min(np.abs(sp - lo32)) > 0.5 * gap * lo and np.min(np.abs(sp - hi32)) > 0.5 * gap * hi
    return lo32, hi32


# ------------------------------------------------------------------- forward

def gpu_fwd(inp, lo, hi):
    io = inp["io"]
    y, hf = ops().ssm_scan_fwd(to_dev(inp["x"], io), to_dev(inp["delta_raw"], io), to_dev(inp["B"], io),
                               to_dev(inp["C"], io), to_dev32(inp["A_log"]), D_skip=to_dev32(inp["D"]),
                               dt_bias=to_dev32(inp["dt_bias"]), z=to_dev(inp["z"], io),
                               h0=to_dev32(inp.get("h0")), dt_min=lo, dt_max=hi)
    torch.cuda.synchronize()
    return host(y), host(hf)


def oracle_fwd(inp, lo, hi):
    return oracle.fwd(inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"], D=inp["D"],
                      dt_bias=inp["dt_bias"], z=inp["z"], h0=inp.get("h0"), dt_min=lo, dt_max=hi)


FWD_CLAMP = [
    ("lanes_fp32", "fwd_b8_l2048_d1536", dict(batch=2, seqlen=300, dim=130, random_h0=True), None),
    ("lanes_bf16", "fwd_bf16_b4_l4096_d4096", dict(batch=2, seqlen=200, dim=96, random_h0=True), None),
    ("lanes_n12", "fwd_b8_l2048_d1536", dict(batch=2, seqlen=77, dim=50, dstate=12), None),
    ("one_state_per_wave_n8", "fwd_b8_l2048_d1536", dict(batch=2, seqlen=150, dim=70, dstate=8), None),
    ("n4", "fwd_b8_l2048_d1536", dict(batch=2, seqlen=90, dim=40, dstate=4), None),
]


@pytest.mark.parametrize("name,wl,over,layout", FWD_CLAMP, ids=[c[0] for c in FWD_CLAMP])
def test_fwd_clamp_parity(name, wl, over, layout):
    inp = W.make_inputs(W.WORKLOADS[wl], **over)
    lo, hi = clamp_bounds(inp)
    say("fwd clamp %s [%.4g, %.4g] B=%d L=%d D=%d N=%d io=%s" % (name, lo, hi, inp["batch"], inp["seqlen"],
                                                                inp["dim"], inp["dstate"], inp["io"]))
    y, hf = gpu_fwd(inp, lo, hi)
    ref = oracle_fwd(inp, lo, hi)
    assert rel_err(y, ref["y"]) <= tol(inp["io"])
    assert rel_err(hf, ref["h_final"]) <= tol(inp["io"])
    # the clamp is active: the unclamped result differs
    free = oracle_fwd(inp, 0.0, float("inf"))
    assert rel_err(free["y"], ref["y"]) > 1e-3


def test_step_clamp_parity():
    inp = W.make_inputs(W.WORKLOADS["step_b256_d5120"], batch=8, dim=300)
    lo, hi = clamp_bounds(inp)
    say("step clamp [%.4g, %.4g]" % (lo, hi))
    st = to_dev32(inp["state"])
    y = ops().ssm_scan_step(st, to_dev32(inp["x"]), to_dev32(inp["delta_raw"]), to_dev32(inp["B"]),
                            to_dev32(inp["C"]), to_dev32(inp["A_log"]), D_skip=to_dev32(inp["D"]),
                            dt_bias=to_dev32(inp["dt_bias"]), z=to_dev32(inp["z"]), dt_min=lo, dt_max=hi)
    torch.cuda.synchronize()
    ref = oracle.step(inp["state"], inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"], D=inp["D"],
                      dt_bias=inp["dt_bias"], z=inp["z"], dt_min=lo, dt_max=hi)
    assert rel_err(host(y), ref["y"]) <= 1e-4
    assert rel_err(host(st), ref["state"]) <= 1e-4


# ------------------------------------------------------------------ backward

def gpu_bwd(inp, lo=None, hi=None, dh_final=None, dh0=True, dy=None):
    g = ops().ssm_scan_bwd(to_dev32(inp["x"]), to_dev32(inp["delta_raw"]), to_dev32(inp["B"]),
                           to_dev32(inp["C"]), to_dev32(inp["A_log"]), to_dev32(inp["dy"] if dy is None else dy),
                           D_skip=to_dev32(inp["D"]), dt_bias=to_dev32(inp["dt_bias"]), z=to_dev32(inp["z"]),
                           h0=to_dev32(inp.get("h0")), dt_min=lo, dt_max=hi, dh_final=to_dev32(dh_final),
                           return_dh0=dh0)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in g.items()}


def oracle_bwd(inp, lo=0.0, hi=float("inf"), dh_final=None):
    return oracle.bwd(inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"], inp["dy"], D=inp["D"],
                      dt_bias=inp["dt_bias"], z=inp["z"], h0=inp.get("h0"), dt_min=lo, dt_max=hi,
                      dh_final=dh_final)


def check(g, r, bound=1e-4):
    bad = {}
    for k in GRADS:
        if r.get(k) is None or g.get(k) is None:
            continue
        e = rel_err(g[k], r[k])
        if not e <= bound:
            bad[k] = e
    assert not bad, bad


BWD_VARIANTS = [
    ("clamp", dict(batch=2, seqlen=130, dim=100, random_h0=True), True, False),
    ("final_state_gradient", dict(batch=2, seqlen=130, dim=100, random_h0=True), False, True),
    ("both", dict(batch=3, seqlen=300, dim=130, random_h0=True), True, True),
    ("many_segments", dict(batch=1, seqlen=3000, dim=64, random_h0=True), True, True),
    ("n5_ungated", dict(batch=2, seqlen=90, dim=70, dstate=5, gated=False), True, True),
    ("seqlen_one", dict(batch=2, seqlen=1, dim=65, random_h0=True), True, True),
    ("wide_rows", dict(batch=2, seqlen=130, dim=64, random_h0=True), True, True),  # 16-byte path
]


@pytest.mark.parametrize("name,over,clamp,final", BWD_VARIANTS, ids=[c[0] for c in BWD_VARIANTS])
def test_bwd_variant_parity(name, over, clamp, final):
    inp = W.make_inputs(W.WORKLOADS["fwdbwd_b4_l2048_d2048"], **over)
    lo, hi = clamp_bounds(inp) if clamp else (None, None)
    dhf = None
    if final:
        rng = np.random.default_rng(17)
        dhf = rng.standard_normal((inp["batch"], inp["dim"], inp["dstate"])).astype(np.float32)
    say("bwd variant %s B=%d L=%d D=%d N=%d clamp=%s dh_final=%s" % (name, inp["batch"], inp["seqlen"],
                                                                     inp["dim"], inp["dstate"], clamp, final))
    g = gpu_bwd(inp, lo, hi, dhf)
    r = oracle_bwd(inp, 0.0 if lo is None else lo, float("inf") if hi is None else hi, dhf)
    check(g, r)
    if clamp:  # steps outside the bounds pass no gradient to delta_raw
        sp = np.logaddexp(0.0, inp["delta_raw"].astype(np.float64) + inp["dt_bias"][None, None, :])
        assert np.all(g["ddelta_raw"][(sp < lo) | (sp > hi)] == 0.0)


def test_bwd_zero_options_are_the_defaults():
    """A zero-initialised options struct (dt_max 0 = no upper bound) and a zero dh_final
    give bit-identical results to no options at all."""
    inp = W.make_inputs(W.WORKLOADS["fwdbwd_b4_l2048_d2048"], batch=2, seqlen=150, dim=90, random_h0=True)
    say("bwd options defaults")
    plain = gpu_bwd(inp, dh0=False)
    zero = gpu_bwd(inp, lo=0.0, hi=0.0, dh_final=np.zeros((2, 90, 16), np.float32), dh0=False)
    for k in GRADS:
        if plain.get(k) is not None:
            assert np.array_equal(plain[k], zero[k]), k


def test_bwd_split_in_two_segments_matches_whole():
    """Backward of [0, L) = backward of [L1, L) from the forward state at L1, then of
    [0, L1) with the second part's dh0 as dh_final (all on the GPU)."""
    inp = W.make_inputs(W.WORKLOADS["fwdbwd_b4_l2048_d2048"], batch=2, seqlen=700, dim=130, random_h0=True)
    L1 = 333
    rng = np.random.default_rng(19)
    dhf = rng.standard_normal((2, 130, 16)).astype(np.float32)
    say("bwd split at %d of %d" % (L1, inp["seqlen"]))
    whole = gpu_bwd(inp, dh_final=dhf)
    seq = ("x", "delta_raw", "z", "B", "C", "dy")
    first = {k: (v[:, :L1] if k in seq and v is not None else v) for k, v in inp.items()}
    second = {k: (v[:, L1:] if k in seq and v is not None else v) for k, v in inp.items()}
    io = inp["io"]
    _, hmid = ops().ssm_scan_fwd(to_dev(first["x"], io), to_dev(first["delta_raw"], io), to_dev(first["B"], io),
                                 to_dev(first["C"], io), to_dev32(inp["A_log"]), D_skip=to_dev32(inp["D"]),
                                 dt_bias=to_dev32(inp["dt_bias"]), z=to_dev(first["z"], io),
                                 h0=to_dev32(inp["h0"]))
    torch.cuda.synchronize()
    second["h0"] = host(hmid)
    g2 = gpu_bwd(second, dh_final=dhf)
    g1 = gpu_bwd(first, dh_final=g2["dh0"])
    for k in ("dx", "ddelta_raw", "dz", "dB", "dC"):
        assert rel_err(np.concatenate([g1[k], g2[k]], 1), whole[k]) <= 1e-4, k
    for k in ("dA_log", "dD", "d_dt_bias"):
        assert rel_err(g1[k] + g2[k], whole[k]) <= 1e-4, k
    assert rel_err(g1["dh0"], whole["dh0"]) <= 1e-4


# ------------------------------------------------------- saved chunk states

def gpu_fwd_save(inp, lo=None, hi=None):
    io = inp["io"]
    b, l, d, n = inp["batch"], inp["seqlen"], inp["dim"], inp["dstate"]
    cs = torch.empty(ops().chunk_states_shape(b, l, d, n), dtype=torch.float32, device="cuda")
    y, hf = ops().ssm_scan_fwd(to_dev(inp["x"], io), to_dev(inp["delta_raw"], io), to_dev(inp["B"], io),
                               to_dev(inp["C"], io), to_dev32(inp["A_log"]), D_skip=to_dev32(inp["D"]),
                               dt_bias=to_dev32(inp["dt_bias"]), z=to_dev(inp["z"], io),
                               h0=to_dev32(inp.get("h0")), dt_min=lo, dt_max=hi, chunk_states=cs)
    torch.cuda.synchronize()
    return host(y), host(hf), cs


@pytest.mark.parametrize("over", [dict(batch=2, seqlen=100, dim=70, random_h0=True),
                                  dict(batch=1, seqlen=48, dim=40, dstate=12)], ids=["n16_ragged", "n12"])
def test_saved_chunk_states_are_the_states_entering_each_chunk(over):
    inp = W.make_inputs(W.WORKLOADS["fwd_b8_l2048_d1536"], **over)
    b, l, d, n = inp["batch"], inp["seqlen"], inp["dim"], inp["dstate"]
    say("fwd saving chunk states B=%d L=%d D=%d N=%d" % (b, l, d, n))
    y, hf, cs = gpu_fwd_save(inp)
    cs = host(cs)                                     # [b, chunk, n, d]
    y0, hf0 = gpu_fwd(inp, None, None)
    assert np.array_equal(y, y0) and np.array_equal(hf, hf0)   # saving changes nothing else
    seq = ("x", "delta_raw", "z", "B", "C")
    for k in range((l + 15) // 16):
        if k == 0:
            ref = inp["h0"] if inp.get("h0") is not None else np.zeros((b, d, n))
        else:
            pre = {kk: (vv[:, : 16 * k] if kk in seq and vv is not None else vv) for kk, vv in inp.items()}
            ref = oracle.fwd(pre["x"], pre["delta_raw"], pre["B"], pre["C"], inp["A_log"], D=inp["D"],
                             dt_bias=inp["dt_bias"], z=pre["z"], h0=inp.get("h0"))["h_final"]
        assert rel_err(cs[:, k].transpose(0, 2, 1), ref) <= 1e-4, k


BWD_SAVED = [
    ("plain", "fwdbwd_b4_l2048_d2048", dict(batch=3, seqlen=300, dim=130, random_h0=True), False, False),
    ("many_segments", "fwdbwd_b4_l2048_d2048", dict(batch=1, seqlen=3000, dim=64, random_h0=True), False, False),
    ("clamp_and_final_gradient", "fwdbwd_b4_l2048_d2048", dict(batch=2, seqlen=200, dim=100, random_h0=True),
     True, True),
    ("bf16", "fwd_bf16_b4_l4096_d4096", dict(batch=2, seqlen=150, dim=96, random_h0=True, with_dy=True),
     False, True),
    ("wide_rows", "fwdbwd_b4_l2048_d2048", dict(batch=2, seqlen=200, dim=64, random_h0=True), True, True),
]


@pytest.mark.parametrize("name,wl,over,clamp,final", BWD_SAVED, ids=[c[0] for c in BWD_SAVED])
def test_bwd_with_saved_chunk_states(name, wl, over, clamp, final):
    inp = W.make_inputs(W.WORKLOADS[wl], **over)
    io = inp["io"]
    lo, hi = clamp_bounds(inp) if clamp else (None, None)
    dhf = np.random.default_rng(23).standard_normal((inp["batch"], inp["dim"], inp["dstate"])).astype(np.float32) \
        if final else None
    say("bwd with saved chunk states %s B=%d L=%d D=%d io=%s" % (name, inp["batch"], inp["seqlen"], inp["dim"], io))
    _, _, cs = gpu_fwd_save(inp, lo, hi)

    def run(states):
        g = ops().ssm_scan_bwd(to_dev(inp["x"], io), to_dev(inp["delta_raw"], io), to_dev(inp["B"], io),
                               to_dev(inp["C"], io), to_dev32(inp["A_log"]), to_dev(inp["dy"], io),
                               D_skip=to_dev32(inp["D"]), dt_bias=to_dev32(inp["dt_bias"]), z=to_dev(inp["z"], io),
                               h0=to_dev32(inp.get("h0")), dt_min=lo, dt_max=hi, dh_final=to_dev32(dhf),
                               return_dh0=True, chunk_states=states)
        torch.cuda.synchronize()
        return {k: (host(v) if v is not None else None) for k, v in g.items()}

    g = run(cs)
    r = oracle_bwd(inp, 0.0 if lo is None else lo, float("inf") if hi is None else hi, dhf)
    check(g, r, tol(io))
    again = run(None)   # the backward that recomputes the states agrees closely
    check(g, again, 1e-5 if io == "fp32" else tol(io))
