"""HIP graph capture of launch-bound sequences.

Short, back-to-back launches (a decode step, the SSD chunk cumsum) are where a HIP
graph pays: the launches replay without host work.  The library enqueues on the
caller's stream and allocates nothing, so a sequence of its calls can be captured with
torch's graph API.  Two sequences are captured once and replayed several times, with
eager work on the same tensors between replays, and every replay is compared bit for
bit with the same calls made eagerly:

  * a decode step: the depthwise conv1d step (its window state updated in place), then
    the selective-scan step on the conv output (its state updated in place);
  * the same decode step as one fused call (ssm_decode_step);
  * the SSD forward pair: the chunk cumsum, then the chunked scan.

No entry point records a memset into the graph (every workspace the kernels read is
written before it is read within the same call).
"""
import numpy as np
import pytest

from _helpers import host, say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from selective_state_space_03_amd import ops
    ops.lib()


def t32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def test_decode_step_graph_replays_match_eager():
    from selective_state_space_03_amd import ops
    from selective_state_space_03_amd import workloads as W
    b, d = 16, 640
    sc = W.make_inputs(W.WORKLOADS["step_b256_d5120"], batch=b, dim=d)
    cv = W.make_conv_inputs(W.CONV_WORKLOADS["conv_step_b256_d5120_k4"], batch=b, dim=d)
    rng = np.random.default_rng(77)
    ntok = 5
    toks = [dict(x=rng.standard_normal((b, d)).astype(np.float32),
                 dr=rng.standard_normal((b, d)).astype(np.float32) - 1.0,
                 B=rng.standard_normal((b, sc["dstate"])).astype(np.float32),
                 C=rng.standard_normal((b, sc["dstate"])).astype(np.float32),
                 z=rng.standard_normal((b, d)).astype(np.float32)) for _ in range(ntok)]
    params = dict(weight=t32(cv["weight"]), bias=t32(cv["bias"]), A_log=t32(sc["A_log"]), D=t32(sc["D"]),
                  dt_bias=t32(sc["dt_bias"]))

    def step(conv_state, ssm_state, x, dr, Bm, Cm, z, u_out, y_out):
        ops.conv1d_step(conv_state, x, params["weight"], bias=params["bias"], silu=True, out=u_out)
        ops.ssm_scan_step(ssm_state, u_out, dr, Bm, Cm, params["A_log"], D_skip=params["D"],
                          dt_bias=params["dt_bias"], z=z, y=y_out)

    # static buffers of the graph, and an eager twin of every state
    st = {k: t32(v) for k, v in dict(x=toks[0]["x"], dr=toks[0]["dr"], B=toks[0]["B"], C=toks[0]["C"],
                                      z=toks[0]["z"]).items()}
    conv_g, ssm_g = t32(cv["state"]), t32(sc["state"])
    conv_e, ssm_e = conv_g.clone(), ssm_g.clone()
    u_g, y_g = torch.empty((b, d), device="cuda"), torch.empty((b, d), device="cuda")
    u_e, y_e = torch.empty_like(u_g), torch.empty_like(y_g)

    # capture on a side stream (warm up once on it first, as graph capture requires);
    # the warm-up step advances the graph's states, so the eager twins take it as well
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(conv_g, ssm_g, st["x"], st["dr"], st["B"], st["C"], st["z"], u_g, y_g)
    torch.cuda.current_stream().wait_stream(s)
    step(conv_e, ssm_e, st["x"], st["dr"], st["B"], st["C"], st["z"], u_e, y_e)
    torch.cuda.synchronize()
    assert torch.equal(conv_g, conv_e) and torch.equal(ssm_g, ssm_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(conv_g, ssm_g, st["x"], st["dr"], st["B"], st["C"], st["z"], u_g, y_g)

    for i, tk in enumerate(toks):
        say("decode graph replay %d" % i)
        for k, key in (("x", "x"), ("dr", "dr"), ("B", "B"), ("C", "C"), ("z", "z")):
            st[k].copy_(t32(tk[key]))
        g.replay()
        step(conv_e, ssm_e, st["x"], st["dr"], st["B"], st["C"], st["z"], u_e, y_e)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), i
        assert torch.equal(conv_g, conv_e) and torch.equal(ssm_g, ssm_e), i
        # eager work on the graph's own buffers between replays
        ssm_g.mul_(1.0)
        torch.cuda.synchronize()
    assert np.isfinite(host(y_g)).all()


def test_fused_decode_step_graph_replays_match_eager():
    from selective_state_space_03_amd import ops
    from selective_state_space_03_amd import workloads as W
    b, d = 16, 640
    sc = W.make_inputs(W.WORKLOADS["step_b256_d5120"], batch=b, dim=d)
    cv = W.make_conv_inputs(W.CONV_WORKLOADS["conv_step_b256_d5120_k4"], batch=b, dim=d)
    rng = np.random.default_rng(78)
    toks = [{k: rng.standard_normal(shp).astype(np.float32) for k, shp in
             (("x", (b, d)), ("dr", (b, d)), ("B", (b, sc["dstate"])), ("C", (b, sc["dstate"])), ("z", (b, d)))}
            for _ in range(4)]
    w, cb = t32(cv["weight"]), t32(cv["bias"])
    A, Dv, dtb = t32(sc["A_log"]), t32(sc["D"]), t32(sc["dt_bias"])

    def step(conv_state, ssm_state, st, y_out):
        ops.decode_step(conv_state, st["x"], w, ssm_state, st["dr"], st["B"], st["C"], A, conv_bias=cb, silu=True,
                        D_skip=Dv, dt_bias=dtb, z=st["z"], y=y_out)

    st = {k: t32(v) for k, v in toks[0].items()}
    conv_g, ssm_g = t32(cv["state"]), t32(sc["state"])
    conv_e, ssm_e = conv_g.clone(), ssm_g.clone()
    y_g, y_e = torch.empty((b, d), device="cuda"), torch.empty((b, d), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(conv_g, ssm_g, st, y_g)
    torch.cuda.current_stream().wait_stream(s)
    step(conv_e, ssm_e, st, y_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(conv_g, ssm_g, st, y_g)
    for i, tk in enumerate(toks):
        say("fused decode graph replay %d" % i)
        for k in st:
            st[k].copy_(t32(tk[k]))
        g.replay()
        step(conv_e, ssm_e, st, y_e)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), i
        assert torch.equal(conv_g, conv_e) and torch.equal(ssm_g, ssm_e), i
        ssm_g.mul_(1.0)  # eager work on the graph's own buffers between replays
        torch.cuda.synchronize()


def test_ssd_forward_graph_replays_match_eager():
    from selective_state_space_03_amd import ops
    from selective_state_space_03_amd import workloads as W
    w = W.SSD_SCAN_WORKLOADS["ssd_scan_small"]
    inp = W.make_ssd_scan_inputs(w, batch=2, seqlen=300, heads=3, dstate=128, h0=True)
    A, dtb, Dv = t32(inp["A"]), t32(inp["dt_bias"]), t32(inp["D"])
    x, Bm, Cm, h0 = t32(inp["x"]), t32(inp["B"]), t32(inp["C"]), t32(inp["h0"])
    dt = t32(inp["dt"])
    b, l, h, p = inp["x"].shape
    n = inp["B"].shape[-1]
    ws = torch.empty((ops.ssd_chunk_scan_fwd_workspace_bytes(b, l, n),), dtype=torch.uint8, device="cuda")

    def pair():
        cs, dto = ops.ssd_chunk_cumsum_fwd(dt, A, w.chunk, dt_bias=dtb)
        y, hf = ops.ssd_chunk_scan_fwd(x, dto, cs, Bm, Cm, D=Dv, h0=h0, workspace=ws)
        return y, hf

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pair()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_g, hf_g = pair()
    rng = np.random.default_rng(5)
    for i in range(3):
        say("ssd graph replay %d" % i)
        dt.copy_(t32(rng.standard_normal(inp["dt"].shape)))
        x.copy_(t32(rng.standard_normal(inp["x"].shape)))
        g.replay()
        y_e, hf_e = pair()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e) and torch.equal(hf_g, hf_e), i
        ws.zero_()  # eager work on a buffer the graph uses; the next replay rewrites it
        torch.cuda.synchronize()
