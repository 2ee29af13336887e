"""GPU parity of the Mamba-2 SSD scan forward (chunk cumsum, then the chunked scan on
the matrix cores) against the fp64 oracle.

y and the final state are compared element by element at max relative error (RMS
floor) <= 1e-4, on shapes with a ragged last chunk, one full chunk, a single step,
d_state 64 and 128, chunks of 64, 128 and 256 steps, with and without the skip term
and an initial state.  The scan is
checked both as a pipeline (the GPU chunk cumsum feeding it) and alone (fed the
oracle's dt_out and dA_cumsum rounded to fp32).  On the full workload (8 x 2048, 64
heads of 64, d_state 128) sampled (batch, head) sequences are compared with the oracle
run on that sequence alone (sequences are independent).  Around the head count at which a
block's x rows reach 2 GB (131071 and 131072 heads of 64), where the scan switches from
16-byte to one-value loads, sampled heads are compared the same way.  The backward is
checked the same way at 131071 and 131072 heads of 64 (its chunk kernel's 16-byte x and
dy loads switch to one-value loads at 2 GB of a chunk's rows) and at 266400 heads of 64,
where one chunk's dy rows span more than 4 GB.  Repeated runs are
bit-identical, and unsupported sizes are refused.
"""
import numpy as np
import pytest

from _helpers import RTOL_F32, host, rel_err, say, to_dev32
from oracle import ssd_cumsum_oracle as CS
from oracle import ssd_scan_oracle as S
from selective_state_space_03_amd import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from selective_state_space_03_amd import ops
    ops.lib()


def oracle_run(inp, bsel=None, hsel=None):
    """fp64 oracle: chunk cumsum for dt_out, then the sequential SSD recurrence"""
    l, w = inp["seqlen"], inp["chunk"]
    dt, A, bias, D, h0 = inp["dt"], inp["A"], inp["dt_bias"], inp["D"], inp["h0"]
    xs, Bs, Cs = inp["x"], inp["B"], inp["C"]
    if bsel is not None:  # one (batch, head) sequence
        hs = slice(hsel, hsel + 1)
        dt, A, bias = dt[bsel:bsel + 1, :, hs], A[hs], bias[hs]
        D = None if D is None else D[hs]
        h0 = None if h0 is None else h0[bsel:bsel + 1, hs]
        xs, Bs, Cs = xs[bsel:bsel + 1, :, hs], Bs[bsel:bsel + 1], Cs[bsel:bsel + 1]
    dA, dto = CS.chunk_cumsum_fwd(dt, A, bias, w, True)
    b, h = dt.shape[0], dt.shape[2]
    flat = dto.transpose(0, 2, 3, 1).reshape(b, -1, h)[:, :l]  # [b, h, nc, w] -> [b, l, h]
    ref = S.ssd_scan_fwd(xs, flat, A, Bs, Cs, D, h0)
    return ref if bsel is not None else (ref, dA, dto)


def gpu_run(inp, cs=None, dto=None):
    from selective_state_space_03_amd import ops
    if cs is None:
        cs, dto = ops.ssd_chunk_cumsum_fwd(to_dev32(inp["dt"]), to_dev32(inp["A"]), inp["chunk"],
                                           dt_bias=to_dev32(inp["dt_bias"]))
    y, hf = ops.ssd_chunk_scan_fwd(to_dev32(inp["x"]), dto, cs, to_dev32(inp["B"]), to_dev32(inp["C"]),
                                   D=to_dev32(inp["D"]), h0=to_dev32(inp["h0"]))
    torch.cuda.synchronize()
    return host(y), host(hf)


CASES = [
    # (batch, seqlen, heads, dstate, skip, h0, chunk)
    (2, 150, 3, 128, True, True, 64),     # ragged last chunk, initial state
    (1, 64, 2, 64, False, False, 64),     # one full chunk, no skip term
    (2, 1, 2, 128, True, True, 64),       # a single step
    (1, 257, 1, 64, True, False, 64),     # five chunks, the last of one step
    (1, 600, 2, 128, True, True, 256),    # 256-step chunks of four blocks, ragged in a middle block
    (2, 300, 1, 64, True, False, 128),    # 128-step chunks, the last block past the end
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_scan_matches_oracle(case):
    b, l, h, n, skip, with_h0, chunk = case
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, batch=b, seqlen=l, heads=h, dstate=n, h0=with_h0, seed=w.seed + l + 7 * n)
    inp["chunk"] = chunk
    if not skip:
        inp["D"] = None
    say("ssd scan b=%d l=%d h=%d n=%d skip=%d h0=%d chunk=%d" % (b, l, h, n, skip, with_h0, chunk))
    ref, rcs, rdto = oracle_run(inp)
    y, hf = gpu_run(inp)
    assert rel_err(y, ref["y"]) <= RTOL_F32
    assert rel_err(hf, ref["h_final"]) <= RTOL_F32
    # the scan alone, fed the oracle's chunk cumsum (rounded to fp32)
    y2, hf2 = gpu_run(inp, cs=to_dev32(rcs), dto=to_dev32(rdto))
    assert rel_err(y2, ref["y"]) <= RTOL_F32
    assert rel_err(hf2, ref["h_final"]) <= RTOL_F32


def test_full_workload_sampled_sequences():
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_b8_l2048_h64_p64_n128"]
    inp = W.make_ssd_scan_inputs(w)
    say("ssd scan full workload %s" % w.name)
    y, hf = gpu_run(inp)
    for (b, h) in ((0, 0), (5, 37), (7, 63)):
        ref = oracle_run(inp, b, h)
        assert rel_err(y[b, :, h], ref["y"][0, :, 0]) <= RTOL_F32
        assert rel_err(hf[b, h], ref["h_final"][0, 0]) <= RTOL_F32



@pytest.mark.parametrize("heads", [131071, 131072])
def test_heads_at_the_wide_load_offset_bound(heads):
    """A 64-step block's x rows span 64 x heads x headdim x 4 bytes.  The 16-byte chunk
    loads address them with 32-bit offsets, so from 2 GB on the scan takes the one-value
    path instead.  131072 heads of 64 are exactly 2 GB and 131071 just below it: sampled
    heads of a two-step sequence against the oracle, on both sides of the bound."""
    from selective_state_space_03_amd import ops
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, batch=1, seqlen=2, heads=heads, dstate=64, seed=w.seed + heads)
    say("ssd scan, %d heads of 64, two steps" % heads)
    cs, dto = ops.ssd_chunk_cumsum_fwd(to_dev32(inp["dt"]), to_dev32(inp["A"]), inp["chunk"],
                                       dt_bias=to_dev32(inp["dt_bias"]))
    y, _ = ops.ssd_chunk_scan_fwd(to_dev32(inp["x"]), dto, cs, to_dev32(inp["B"]), to_dev32(inp["C"]),
                                  D=to_dev32(inp["D"]), h_final=None)
    torch.cuda.synchronize()
    y = host(y)
    for h in (0, 77777, heads - 1):
        ref = oracle_run(inp, 0, h)
        assert rel_err(y[0, :, h], ref["y"][0, :, 0]) <= RTOL_F32, h

def test_repeat_runs_are_bit_identical():
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, h0=True)
    runs = [gpu_run(inp) for _ in range(3)]
    for y, hf in runs[1:]:
        assert y.tobytes() == runs[0][0].tobytes() and hf.tobytes() == runs[0][1].tobytes()


@pytest.mark.parametrize("dstate", [128, 64])
def test_wide_and_narrow_chunk_loads_agree_bit_for_bit(dstate):
    """With x, B and C 16-byte aligned the scan loads each chunk as 16-byte pieces; an x
    that is not 16-byte aligned sends the same call down the one-value path.  The staged
    tiles and every product are the same, so y, the final state and the saved block
    states must be bit-identical."""
    from selective_state_space_03_amd import ops
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, batch=2, seqlen=300, heads=3, dstate=dstate, h0=True)
    say("ssd scan wide vs narrow chunk loads, d_state %d" % dstate)
    cs, dto = ops.ssd_chunk_cumsum_fwd(to_dev32(inp["dt"]), to_dev32(inp["A"]), inp["chunk"],
                                       dt_bias=to_dev32(inp["dt_bias"]))
    x = to_dev32(inp["x"])
    buf = torch.zeros(x.numel() + 1, dtype=torch.float32, device="cuda")
    x_odd = buf[1:].view(x.shape)  # contiguous, 4 bytes past a 16-byte boundary
    x_odd.copy_(x)
    b, l, h, p = inp["x"].shape
    outs = []
    for xx in (x, x_odd):
        bs = torch.empty(ops.ssd_block_states_shape(b, l, h, p, dstate), dtype=torch.float32, device="cuda")
        y, hf = ops.ssd_chunk_scan_fwd(xx, dto, cs, to_dev32(inp["B"]), to_dev32(inp["C"]), D=to_dev32(inp["D"]),
                                       h0=to_dev32(inp["h0"]), block_states=bs)
        torch.cuda.synchronize()
        outs.append((host(y), host(hf), host(bs)))
    for a_, b_ in zip(outs[0], outs[1]):
        assert np.array_equal(a_, b_)


def test_unsupported_sizes_are_refused():
    from selective_state_space_03_amd import ops
    dev = "cuda"
    x = torch.zeros((1, 64, 1, 32), device=dev)           # headdim 32
    ch = torch.zeros((1, 1, 1, 64), device=dev)
    bc = torch.zeros((1, 64, 128), device=dev)
    with pytest.raises(ops.SsmError):
        ops.ssd_chunk_scan_fwd(x, ch, ch, bc, bc)
    x = torch.zeros((1, 64, 1, 64), device=dev)
    with pytest.raises(ops.SsmError):
        ops.ssd_chunk_scan_fwd(x, ch, ch, torch.zeros((1, 64, 96), device=dev), torch.zeros((1, 64, 96), device=dev))
    ch32 = torch.zeros((1, 1, 2, 32), device=dev)           # chunk 32
    with pytest.raises(ops.SsmError):
        ops.ssd_chunk_scan_fwd(x, ch32, ch32, bc, bc)
    ch96 = torch.zeros((1, 1, 1, 96), device=dev)           # chunk 96, not a multiple of 64
    with pytest.raises(ops.SsmError):
        ops.ssd_chunk_scan_fwd(x, ch96, ch96, bc, bc)


# ------------------------------------------------------------------ backward

def oracle_bwd(inp, dy, dhf):
    """fp64 oracle of the whole pipeline's gradients: the sequential adjoint of the scan
    with respect to dt_out, then through softplus to the raw dt (no clamp binds)"""
    from oracle import ssd_cumsum_oracle as CSo
    l, w = inp["seqlen"], inp["chunk"]
    _, dto = CSo.chunk_cumsum_fwd(inp["dt"], inp["A"], inp["dt_bias"], w, True)
    b, h = inp["dt"].shape[0], inp["dt"].shape[2]
    flat = dto.transpose(0, 2, 3, 1).reshape(b, -1, h)[:, :l]
    g = S.ssd_scan_bwd(inp["x"], flat, inp["A"], inp["B"], inp["C"], dy, inp["D"], inp["h0"], dhf)
    raw = inp["dt"].astype(np.float64) + inp["dt_bias"].astype(np.float64)[None, None]
    g["ddt_raw"] = g["ddt"] * CSo._g_prime(raw, True)
    g["d_dt_bias"] = g["ddt_raw"].sum(axis=(0, 1))
    return g


def gpu_bwd(inp, dy, dhf):
    from selective_state_space_03_amd import ops
    dt, A, bias = to_dev32(inp["dt"]), to_dev32(inp["A"]), to_dev32(inp["dt_bias"])
    cs, dto = ops.ssd_chunk_cumsum_fwd(dt, A, inp["chunk"], dt_bias=bias)
    b, l, h, p = inp["x"].shape
    n = inp["B"].shape[-1]
    bs = torch.empty(ops.ssd_block_states_shape(b, l, h, p, n), dtype=torch.float32, device="cuda")
    x, Bm, Cm, D = to_dev32(inp["x"]), to_dev32(inp["B"]), to_dev32(inp["C"]), to_dev32(inp["D"])
    ops.ssd_chunk_scan_fwd(x, dto, cs, Bm, Cm, D=D, h0=to_dev32(inp["h0"]), block_states=bs)
    g = ops.ssd_chunk_scan_bwd(x, dto, cs, Bm, Cm, to_dev32(dy), bs, D=D, dh_final=to_dev32(dhf), return_dh0=True)
    gc = ops.ssd_chunk_cumsum_bwd(g["ddA_cumsum"], g["ddt_out"], dt, A, dt_bias=bias)
    torch.cuda.synchronize()
    out = {k: (None if v is None else host(v)) for k, v in g.items()}
    out.update(ddt_raw=host(gc["ddt"]), dA=host(gc["dA"]), d_dt_bias=host(gc["d_dt_bias"]))
    return out


BWD_CASES = [
    # (batch, seqlen, heads, dstate, skip, h0, dh_final)
    (2, 150, 3, 128, True, True, True),    # ragged last chunk, initial state and final-state gradient
    (1, 64, 2, 64, False, False, False),   # one full chunk, no skip term
    (2, 1, 2, 128, True, True, False),     # a single step
    (1, 257, 1, 64, True, False, True),    # five chunks, the last of one step
    (2, 512, 4, 128, True, True, True),    # eight chunks
    (3, 1300, 11, 64, True, True, True),   # heads of a chunk in uneven groups (3, 3, 3, 2), ragged chunk
    (4, 4096, 2, 64, False, True, True),   # 256 (batch, chunk) pairs: every head in one group
    (4, 4050, 2, 128, True, False, True),  # one group, d_state 128, a ragged last chunk of 18 steps
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(i) for i in range(len(BWD_CASES))])
def test_scan_backward_matches_oracle(case):
    b, l, h, n, skip, with_h0, with_dhf = case
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, batch=b, seqlen=l, heads=h, dstate=n, h0=with_h0, seed=w.seed + 3 * l + n)
    if not skip:
        inp["D"] = None
    rng = np.random.default_rng(w.seed + l)
    dy = rng.standard_normal(inp["x"].shape).astype(np.float32)
    dhf = rng.standard_normal((b, h, 64, n)).astype(np.float32) if with_dhf else None
    say("ssd scan bwd b=%d l=%d h=%d n=%d skip=%d h0=%d dhf=%d" % (b, l, h, n, skip, with_h0, with_dhf))
    g = gpu_bwd(inp, dy, dhf)
    r = oracle_bwd(inp, dy, dhf)
    bad = {}
    for k_gpu, k_ref in (("dx", "dx"), ("dB", "dB"), ("dC", "dC"), ("dD", "dD"), ("dh0", "dh0"),
                         ("ddt_raw", "ddt_raw"), ("dA", "dA"), ("d_dt_bias", "d_dt_bias")):
        e = rel_err(g[k_gpu], r[k_ref])
        if not e <= RTOL_F32:
            bad[k_gpu] = e
    assert not bad, bad


def test_scan_backward_is_bit_identical_across_runs():
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, h0=True)
    dy = np.random.default_rng(5).standard_normal(inp["x"].shape).astype(np.float32)
    runs = [gpu_bwd(inp, dy, None) for _ in range(3)]
    for r in runs[1:]:
        for k, v in r.items():
            if v is not None:
                assert v.tobytes() == runs[0][k].tobytes(), k



@pytest.mark.parametrize("dstate", [128, 64])
def test_backward_wide_and_narrow_loads_agree_bit_for_bit(dstate):
    """With x, dy, B, C and the block states 16-byte aligned the backward's chunk kernel
    loads them as 16-byte pieces; a dy that is not 16-byte aligned sends the same call
    down the one-value path.  The staged tiles are the same and both paths take the
    entering state in the same pieces, so every output must be bit-identical."""
    from selective_state_space_03_amd import ops
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, batch=2, seqlen=300, heads=5, dstate=dstate, h0=True)
    say("ssd scan bwd wide vs narrow loads, d_state %d" % dstate)
    cs, dto = ops.ssd_chunk_cumsum_fwd(to_dev32(inp["dt"]), to_dev32(inp["A"]), inp["chunk"],
                                       dt_bias=to_dev32(inp["dt_bias"]))
    b, l, h, p = inp["x"].shape
    x, Bm, Cm, D = to_dev32(inp["x"]), to_dev32(inp["B"]), to_dev32(inp["C"]), to_dev32(inp["D"])
    bs = torch.empty(ops.ssd_block_states_shape(b, l, h, p, dstate), dtype=torch.float32, device="cuda")
    ops.ssd_chunk_scan_fwd(x, dto, cs, Bm, Cm, D=D, h0=to_dev32(inp["h0"]), block_states=bs)
    rng = np.random.default_rng(w.seed + 17)
    dy = to_dev32(rng.standard_normal(inp["x"].shape))
    dhf = to_dev32(rng.standard_normal((b, h, p, dstate)))
    buf = torch.zeros(dy.numel() + 1, dtype=torch.float32, device="cuda")
    dy_odd = buf[1:].view(dy.shape)  # contiguous, 4 bytes past a 16-byte boundary
    dy_odd.copy_(dy)
    outs = []
    for d in (dy, dy_odd):
        g = ops.ssd_chunk_scan_bwd(x, dto, cs, Bm, Cm, d, bs, D=D, dh_final=dhf, return_dh0=True)
        torch.cuda.synchronize()
        outs.append({k: host(v) for k, v in g.items() if v is not None})
    assert outs[0].keys() == outs[1].keys()
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k

def test_scan_backward_full_workload_sampled_sequences():
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_b8_l2048_h64_p64_n128"]
    inp = W.make_ssd_scan_inputs(w)
    dy = np.random.default_rng(w.seed).standard_normal(inp["x"].shape, dtype=np.float32)
    say("ssd scan bwd full workload %s" % w.name)
    g = gpu_bwd(inp, dy, None)
    for (b, h) in ((0, 0), (6, 41)):
        one = {"seqlen": inp["seqlen"], "chunk": inp["chunk"], "dt": inp["dt"][b:b + 1, :, h:h + 1],
               "A": inp["A"][h:h + 1], "dt_bias": inp["dt_bias"][h:h + 1], "x": inp["x"][b:b + 1, :, h:h + 1],
               "B": inp["B"][b:b + 1], "C": inp["C"][b:b + 1], "D": inp["D"][h:h + 1], "h0": None}
        r = oracle_bwd(one, dy[b:b + 1, :, h:h + 1], None)
        assert rel_err(g["dx"][b, :, h], r["dx"][0, :, 0]) <= RTOL_F32
        assert rel_err(g["dh0"][b, h], r["dh0"][0, 0]) <= RTOL_F32
        assert rel_err(g["ddt_raw"][b, :, h], r["ddt_raw"][0, :, 0]) <= RTOL_F32



@pytest.mark.parametrize("heads", [131071, 131072])
def test_scan_backward_heads_at_the_wide_load_offset_bound(heads):
    """The chunk kernel's 16-byte x and dy loads address a chunk's rows with 32-bit byte
    offsets from the head's first row, so from 2 GB of rows (131072 heads of 64) on, the
    backward takes the one-value path.  Both sides of the bound, a two-step sequence:
    dx, dh0 and the raw step gradient of sampled heads against the oracle."""
    from selective_state_space_03_amd import ops
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, batch=1, seqlen=2, heads=heads, dstate=64, seed=w.seed + heads)
    b, l, h, p = inp["x"].shape
    n = inp["B"].shape[-1]
    dy = np.random.default_rng(heads).standard_normal(inp["x"].shape).astype(np.float32)
    say("ssd scan bwd, %d heads of 64, two steps" % heads)
    dt, A, dtb = to_dev32(inp["dt"]), to_dev32(inp["A"]), to_dev32(inp["dt_bias"])
    cs, dto = ops.ssd_chunk_cumsum_fwd(dt, A, inp["chunk"], dt_bias=dtb)
    x, Bd, Cd, Dd = to_dev32(inp["x"]), to_dev32(inp["B"]), to_dev32(inp["C"]), to_dev32(inp["D"])
    bs = torch.empty(ops.ssd_block_states_shape(b, l, h, p, n), dtype=torch.float32, device="cuda")
    ops.ssd_chunk_scan_fwd(x, dto, cs, Bd, Cd, D=Dd, h_final=None, block_states=bs)
    g = ops.ssd_chunk_scan_bwd(x, dto, cs, Bd, Cd, to_dev32(dy), bs, D=Dd, return_dh0=True)
    gc = ops.ssd_chunk_cumsum_bwd(g["ddA_cumsum"], g["ddt_out"], dt, A, dt_bias=dtb)
    torch.cuda.synchronize()
    for hh in (0, 77777, h - 1):
        one = {"seqlen": l, "chunk": inp["chunk"], "dt": inp["dt"][:, :, hh:hh + 1], "A": inp["A"][hh:hh + 1],
               "dt_bias": inp["dt_bias"][hh:hh + 1], "x": inp["x"][:, :, hh:hh + 1], "B": inp["B"], "C": inp["C"],
               "D": inp["D"][hh:hh + 1], "h0": None}
        r = oracle_bwd(one, dy[:, :, hh:hh + 1], None)
        assert rel_err(host(g["dx"][:, :, hh]), r["dx"][:, :, 0]) <= RTOL_F32, hh
        assert rel_err(host(g["dh0"][:, hh]), r["dh0"][:, 0]) <= RTOL_F32, hh
        assert rel_err(host(gc["ddt"][:, :, hh]), r["ddt_raw"][:, :, 0]) <= RTOL_F32, hh


def test_scan_backward_rows_more_than_4gb_apart_in_a_chunk():
    """dy rows of one chunk are heads x headdim x 4 bytes apart.  At 266400 heads of 64 a
    full chunk's 64 rows span more than 4 GB, past any 32-bit offset from the chunk's
    first row.  One full chunk; x and dy (1.1 G values each) are drawn on the device from
    a seeded generator, the rest on the host.  Sampled heads are compared with the oracle
    run on that head alone."""
    from selective_state_space_03_amd import ops
    b, l, h, p, n, chunk = 1, 64, 266400, 64, 64, 64
    assert 63 * h * p * 4 >= 1 << 32
    rng = np.random.default_rng(4242)
    dt = rng.standard_normal((b, l, h)).astype(np.float32)
    dt_bias = np.log(np.expm1(rng.uniform(1e-3, 1e-1, h))).astype(np.float32)
    A = (-rng.uniform(1.0, 16.0, h)).astype(np.float32)
    Bm = rng.standard_normal((b, l, n)).astype(np.float32)
    Cm = rng.standard_normal((b, l, n)).astype(np.float32)
    D = np.ones(h, np.float32)
    gen = torch.Generator(device="cuda").manual_seed(4243)
    x = torch.randn((b, l, h, p), generator=gen, device="cuda")
    dy = torch.randn((b, l, h, p), generator=gen, device="cuda")
    say("ssd scan bwd, %d heads of 64, one chunk" % h)
    cs, dto = ops.ssd_chunk_cumsum_fwd(to_dev32(dt), to_dev32(A), chunk, dt_bias=to_dev32(dt_bias))
    Bd, Cd, Dd = to_dev32(Bm), to_dev32(Cm), to_dev32(D)
    bs = torch.empty(ops.ssd_block_states_shape(b, l, h, p, n), dtype=torch.float32, device="cuda")
    ops.ssd_chunk_scan_fwd(x, dto, cs, Bd, Cd, D=Dd, h_final=None, block_states=bs)
    g = ops.ssd_chunk_scan_bwd(x, dto, cs, Bd, Cd, dy, bs, D=Dd, return_dh0=True)
    gc = ops.ssd_chunk_cumsum_bwd(g["ddA_cumsum"], g["ddt_out"], to_dev32(dt), to_dev32(A), dt_bias=to_dev32(dt_bias))
    torch.cuda.synchronize()
    for hh in (0, 123457, h - 1):
        one = {"seqlen": l, "chunk": chunk, "dt": dt[:, :, hh:hh + 1], "A": A[hh:hh + 1],
               "dt_bias": dt_bias[hh:hh + 1], "x": host(x[:, :, hh:hh + 1]), "B": Bm, "C": Cm,
               "D": D[hh:hh + 1], "h0": None}
        r = oracle_bwd(one, host(dy[:, :, hh:hh + 1]), None)
        assert rel_err(host(g["dx"][:, :, hh]), r["dx"][:, :, 0]) <= RTOL_F32, hh
        assert rel_err(host(g["dh0"][:, hh]), r["dh0"][:, 0]) <= RTOL_F32, hh
        assert rel_err(host(gc["ddt"][:, :, hh]), r["ddt_raw"][:, :, 0]) <= RTOL_F32, hh

def test_scan_backward_full_length_all_heads_one_batch_element():
    """Every output of the backward at the workload's per-sequence size (L = 2048,
    64 heads of 64, d_state 128, one batch element), including the sums over heads
    (dB, dC: one writer per element, as in deterministic_backward.py's
    single_writer_kernels, the heads added in a fixed order) and over time (dD, dA,
    d_dt_bias), against the sequential fp64 adjoint."""
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_b8_l2048_h64_p64_n128"]
    inp = W.make_ssd_scan_inputs(w, batch=1)
    dy = np.random.default_rng(w.seed + 11).standard_normal(inp["x"].shape, dtype=np.float32)
    say("ssd scan bwd b=1 l=%d h=%d n=%d (all outputs)" % (inp["seqlen"], inp["heads"], inp["dstate"]))
    g = gpu_bwd(inp, dy, None)
    say("ssd scan bwd b=1: oracle")
    r = oracle_bwd(inp, dy, None)
    bad = {}
    for k in ("dx", "dB", "dC", "dD", "dh0", "ddt_raw", "dA", "d_dt_bias"):
        e = rel_err(g[k], r[k])
        if not e <= RTOL_F32:
            bad[k] = e
    assert not bad, bad
