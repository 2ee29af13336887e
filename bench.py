"""Benchmark of the gfx950 selective-scan hot path on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                  [--only fwd|bf16|long|step|decode|fwd5|bwd|bwd_bf16|train|mamba3|ssd|conv|conv_bf16|conv_step|conv_bwd|copy]

Timed step: one forward scan of the workload B=8, L=2048, d_inner=1536, N=16, fp32
I/O, SiLU gate (x, delta_raw, z, B, C, A_log, D_skip, dt_bias in HBM; y and the
final state written).  W untimed warmups, then exactly K timed steps between two
device synchronisations.  Inputs are seeded synthetic tensors (workloads.py),
resident in HBM before timing; several identical buffer sets are rotated so that
every step streams from HBM rather than from the 256 MB last-level cache.

Printed: ONE JSON line on stdout (everything else goes to stderr) with the
headline forward GB/s, its roofline (algorithmic bytes per launch / average launch
time from HIP events on the launch stream, against 8 TB/s), the fp64 CPU oracle
timed on the host cores, and secondary lines for the bf16 forward, the decode
step (alone, and fused with the conv1d step), the backward, the conv1d, the Mamba-3 preprocess adjoint and the Mamba-2 SSD
chunk cumsum and scan (the scan also in TFLOP/s against the fp32 matrix-core
peak).  `traffic` comes from the committed rocprofv3 counter
summary for the forward kernel when that summary matches the current kernel
source, else null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# VALU issue rate of fp32 non-packed instructions: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
# minimal issue slots per state update: mul (Delta*A), exp2 (half rate = 2 slots),
# mul (Delta*x*B), fma (state), fma (readout)
SLOTS_PER_UPDATE = 6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_bytes(b, l, d, n, es, gated, h_final=True):
    E, S, H = b * l * d, b * l * n, b * d * n
    return (E * es * (3 if gated else 2) + E * es + 2 * S * es + (H * 4 if h_final else 0)
            + d * n * 4 + 2 * d * 4)


def step_bytes(b, d, n, es, gated):
    E, H = b * d, b * d * n
    return 2 * H * 4 + E * es * (3 if gated else 2) + E * es + 2 * b * n * es + d * n * 4 + 2 * d * 4


def bwd_bytes(b, l, d, n, gated, es=4):
    """activations (x, delta_raw, z, dy in; dx, ddelta_raw, dz out) and B, C at the I/O
    size es; dB, dC and the parameter gradients in fp32"""
    E, S = b * l * d, b * l * n
    reads = E * es * (4 if gated else 3) + 2 * S * es + d * n * 4 + 2 * d * 4
    writes = E * es * (3 if gated else 2) + 2 * S * 4 + d * n * 4 + 2 * d * 4
    return reads + writes


def mamba3_bytes(rows, inner, state, heads, angles, bc):
    """Mamba-3 preprocess adjoint: the read parts of the projected rows (B, C, dd_dt,
    dd_a) and dt_bias, every incoming gradient, the written gradient row, the row
    partials and d_dt_bias (fp32)"""
    width = 2 * inner + 2 * bc * state + 3 * heads + angles
    reads = rows * (2 * bc * state + 2 * heads) + heads + rows * (2 * inner + 2 * bc * state + 3 * heads + angles)
    writes = rows * width + rows * heads + heads
    return 4 * (reads + writes)


def ssd_fwd_bytes(b, l, h, nc, w):
    """SSD chunk cumsum: dt read, A and dt_bias read, dA_cumsum and dt_out written (fp32)"""
    return 4 * (b * l * h + 2 * h + 2 * b * h * nc * w)


def ssd_bwd_bytes(b, l, h, nc, w):
    """its backward: ddA, ddt_out, dt, A, dt_bias read; ddt, dA, d_dt_bias written (fp32)"""
    return 4 * (2 * b * h * nc * w + b * l * h + 2 * h + b * l * h + 2 * h)


def ssd_scan_bytes(b, l, h, p, n, nc, w):
    """SSD scan forward: x read, y written, B and C read once, dt_out and dA_cumsum read,
    D read (fp32)"""
    return 4 * (2 * b * l * h * p + 2 * b * l * n + 2 * b * h * nc * w + h)


def ssd_scan_flops(b, l, h, p, n, nc, w):
    """useful multiply-adds of the chunked form, x2: per (batch, head, chunk) the
    inter-chunk readout C S^T (w n p), the causal M X (w (w + 1) / 2 pairs, p each) and
    the state update X^T B (w p n); per (batch, chunk) the causal C B^T (w (w + 1) / 2
    pairs, n each), which the heads share (one B, C group)"""
    tri = w * (w + 1) // 2
    return 2 * b * h * nc * (w * n * p + tri * p + w * p * n) + 2 * b * nc * tri * n


def ssd_scan_bwd_bytes(b, l, h, p, n, nc, w):
    """SSD scan backward: x, dy read and dx written, B and C read once and dB, dC written,
    dt_out and dA_cumsum read and their gradients written, the saved block states read,
    dh0 written (fp32)"""
    return 4 * (3 * b * l * h * p + 4 * b * l * n + 4 * b * h * nc * w + b * h * nc * p * n + b * h * p * n)


def ssd_scan_bwd_flops(b, l, h, p, n, nc, w):
    """useful multiply-adds of the chunked backward, x2: per (batch, head, chunk) five
    full products of w p n (B G^T, X G, dY S, C S^T and the carry update) and the causal
    dY X^T and K^T dY (w (w + 1) / 2 pairs each, of length p); per (batch, chunk), since
    B and C are shared by the heads, the causal C B^T once and the V terms V B and V^T C
    once on V summed over the heads (w (w + 1) / 2 pairs each, of length n)"""
    tri = w * (w + 1) // 2
    return 2 * b * h * nc * (5 * w * p * n + tri * 2 * p) + 2 * b * nc * tri * 3 * n


def conv_bytes(b, l, d, k, es):
    """depthwise causal conv1d: x read, out written, weight and bias read"""
    return 2 * b * l * d * es + d * k * 4 + d * 4


def conv_step_bytes(b, d, k, es):
    """one decode step: state read and written, x read, out written, weight and bias read"""
    return 2 * b * d * (k - 1) * es + 2 * b * d * es + d * k * 4 + d * 4


def decode_bytes(b, d, n, k, es, gated):
    """the fused decode step: the scan step's and the conv1d step's bytes, less the
    convolution's output, which neither writes nor reads (x enters the convolution)"""
    return step_bytes(b, d, n, es, gated) + conv_step_bytes(b, d, k, es) - 2 * b * d * es


def conv_bwd_bytes(b, l, d, k):
    """x and dout read, dx written; weight and bias read, their gradients written"""
    return 3 * b * l * d * 4 + 2 * (d * k * 4 + d * 4)


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


FWD_SOURCES = ["selective_state_space_03_amd/csrc/ssm_fwd.hip", "selective_state_space_03_amd/csrc/ssm_device.h"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fwd_b8_l2048_d1536_counters.json")


def measured_traffic():
    """HBM bytes per launch of the forward kernel from the committed counter summary,
    or None if absent or taken on a different kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_digest") != source_digest(FWD_SOURCES):
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_model():
    """the host CPU's model name (lscpu), or None"""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


def cpu_baseline(head):
    """The fp64 oracle timed on the host, on the same synthetic inputs as the GPU lines:
    every forward workload, the decode step and the backward on the oracle's thread pool
    (the machine's CPU share, at most 16 threads), plus the small and the benchmark forward
    on one thread.  Whole passes are timed; the benchmark forward is repeated until about
    10 s are spent on it.  The headline value is the benchmark forward's GB/s."""
    import oracle
    from selective_state_space_03_amd import workloads as W
    nthreads = oracle.default_threads()
    per = {}

    def timed(fn, min_s=0.0):
        passes, t0 = 0, time.perf_counter()
        while passes == 0 or time.perf_counter() - t0 < min_s:
            fn()
            passes += 1
        return (time.perf_counter() - t0) / passes, passes

    def fwd_of(inp, nt):
        return lambda: oracle.fwd(inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"], D=inp["D"],
                                  dt_bias=inp["dt_bias"], z=inp["z"], nthreads=nt)

    for name in ("fwd_small", "fwd_b8_l2048_d1536", "fwd_bf16_b4_l4096_d4096", "fwdbwd_b4_l2048_d2048"):
        w = W.WORKLOADS[name]
        inp = head["inp"] if name == "fwd_b8_l2048_d1536" else W.make_inputs(w, with_dy=False)
        es = 2 if w.io == "bf16" else 4
        nb = fwd_bytes(w.batch, w.seqlen, w.dim, w.dstate, es, w.gated)
        dt, passes = timed(fwd_of(inp, nthreads), 10.0 if name == "fwd_b8_l2048_d1536" else 0.0)
        per["fwd_" + name] = {"seconds_per_pass": round(dt, 5), "passes": passes, "threads": nthreads,
                              "gbs": round(nb / dt / 1e9, 4), "elements_per_s": round(w.elements / dt, 1)}
        if name in ("fwd_small", "fwd_b8_l2048_d1536"):
            dt1, p1 = timed(fwd_of(inp, 1))
            per["fwd_" + name + "_1thread"] = {"seconds_per_pass": round(dt1, 5), "passes": p1, "threads": 1,
                                               "gbs": round(nb / dt1 / 1e9, 4)}
        log("cpu oracle fwd %-24s %.4f s per pass on %d threads" % (name, dt, nthreads))
    w = W.WORKLOADS["step_b256_d5120"]
    inp = W.make_inputs(w)
    dt, passes = timed(lambda: oracle.step(inp["state"], inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"],
                                           D=inp["D"], dt_bias=inp["dt_bias"], z=inp["z"], nthreads=nthreads), 1.0)
    per["step_b256_d5120"] = {"seconds_per_pass": round(dt, 5), "passes": passes, "threads": nthreads,
                              "gbs": round(step_bytes(w.batch, w.dim, w.dstate, 4, w.gated) / dt / 1e9, 4)}
    w = W.WORKLOADS["fwdbwd_b4_l2048_d2048"]
    inp = W.make_inputs(w)
    dt, passes = timed(lambda: oracle.bwd(inp["x"], inp["delta_raw"], inp["B"], inp["C"], inp["A_log"], inp["dy"],
                                          D=inp["D"], dt_bias=inp["dt_bias"], z=inp["z"], nthreads=nthreads))
    per["bwd_b4_l2048_d2048"] = {"seconds_per_pass": round(dt, 5), "passes": passes, "threads": nthreads,
                                 "gbs": round(bwd_bytes(w.batch, w.seqlen, w.dim, w.dstate, w.gated) / dt / 1e9, 4)}
    log("cpu oracle step %.4f s, bwd %.4f s per pass" % (per["step_b256_d5120"]["seconds_per_pass"], dt))
    hb = per["fwd_fwd_b8_l2048_d1536"]
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"value": hb["gbs"], "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": "the fp64 oracle on the same inputs: %d whole passes of the benchmark forward (B=8 L=2048 "
                      "d_inner=1536 N=16), one pass of each other forward workload, the decode step and the backward "
                      "on %d threads, and the small and benchmark forwards on 1 thread" % (hb["passes"], nthreads),
            "seconds_per_pass": hb["seconds_per_pass"], "gpu_speedup": round(hb["seconds_per_pass"] / (head["ev_ms"] * 1e-3), 1),
            "threads": nthreads, "host_cpu_count": os.cpu_count(), "host_affinity_cpus": aff, "host_cpu_model": cpu_model(),
            "per_workload": per}


class Timer:
    """HIP events on the current (launch) stream, which is the stream the library
    launches on.  The average launch duration is one event pair around the K timed
    launches, divided by K: the launches queue back to back, so it is the kernels'
    time plus the gaps between them, with no event record between two launches.  The
    minimum comes from a few more launches with a pair each, outside that region."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps, warmup, nsets):
        torch = self.torch
        for i in range(warmup):
            fn(i % nsets)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            fn(i % nsets)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        avg = start.elapsed_time(end) / steps  # ms
        n_min = min(steps, 10)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_min)]
        for i in range(n_min):
            evs[i][0].record()
            fn(i % nsets)
            evs[i][1].record()
        torch.cuda.synchronize()
        return wall * 1e3 / steps, avg, min(a.elapsed_time(b) for a, b in evs)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all",
                    choices=["all", "fwd", "bf16", "long", "step", "decode", "fwd5", "bwd", "bwd_bf16", "train", "mamba3", "conv", "conv_bf16", "conv_step", "conv_bwd",
                             "ssd", "copy"])
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the selective scan here has no multi-GPU path "
              "(each GPU would run the same kernels on its own batch rows or channel slices); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from selective_state_space_03_amd import ops
    from selective_state_space_03_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops.lib()
    timer = Timer(torch)
    K, Wm = args.steps, args.warmup
    results = {}

    def t32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    def tio(a, io):
        t = t32(a)
        return t.to(torch.bfloat16) if (t is not None and io == "bf16") else t

    def direct(fname, *args):
        """The C entry point with its arguments marshalled once.  Used for launches of a
        few microseconds, where the binding's per-call Python checks would take longer
        than the kernel and the events would time them instead; every set is first run
        once through the checked binding."""
        f = getattr(ops.lib(), fname)
        cargs = [ops._ptr(a) if isinstance(a, torch.Tensor) else a for a in args]

        def call():
            st = f(*cargs)
            if st != 0:
                raise RuntimeError("%s returned %d" % (fname, st))
        return call

    def fwd_case(name, min_bytes_rotation=1.2e9, save=False):
        # save: also write the chunk states for the backward (same algorithmic bytes;
        # the states are an implementation overhead of the training path)
        w = W.WORKLOADS[name]
        inp = W.make_inputs(w, with_dy=False)
        io = w.io
        es = 2 if io == "bf16" else 4
        nb = fwd_bytes(w.batch, w.seqlen, w.dim, w.dstate, es, w.gated)
        nsets = max(2, int(np.ceil(min_bytes_rotation / nb)))
        base = dict(x=tio(inp["x"], io), dr=tio(inp["delta_raw"], io), z=tio(inp["z"], io), B=tio(inp["B"], io),
                    C=tio(inp["C"], io))
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        A_log, Dsk, dtb = t32(inp["A_log"]), t32(inp["D"]), t32(inp["dt_bias"])
        ys = [torch.empty_like(base["x"]) for _ in range(nsets)]
        hfs = [torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev) for _ in range(nsets)]
        css = [torch.empty(ops.chunk_states_shape(w.batch, w.seqlen, w.dim, w.dstate), dtype=torch.float32,
                           device=dev) if save else None for _ in range(nsets)]
        # the time-split path (long sequences of few channels) takes a workspace
        wsb = ops.fwd_workspace_bytes(w.batch, w.seqlen, w.dim, w.dstate, ops.SSM_BF16 if io == "bf16" else ops.SSM_F32)
        wss = [torch.empty((wsb,), dtype=torch.uint8, device=dev) if wsb else None for _ in range(nsets)]

        def fn(i):
            s = sets[i]
            ops.ssm_scan_fwd(s["x"], s["dr"], s["B"], s["C"], A_log, D_skip=Dsk, dt_bias=dtb, z=s["z"],
                             y=ys[i], h_final=hfs[i], chunk_states=css[i], workspace=wss[i])

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f%% of 8 TB/s  sets=%d" %
            (name + ("_save" if save else ""), ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, nsets))
        return dict(workload=w, bytes=nb, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs,
                    wall_gbs=nb / (wall_ms * 1e-3) / 1e9, inp=inp)

    def step_case(name="step_b256_d5120"):
        w = W.WORKLOADS[name]
        inp = W.make_inputs(w)
        nb = step_bytes(w.batch, w.dim, w.dstate, 4, w.gated)
        nsets = max(2, int(np.ceil(1.2e9 / nb)))
        base = dict(st=t32(inp["state"]), x=t32(inp["x"]), dr=t32(inp["delta_raw"]), z=t32(inp["z"]),
                    B=t32(inp["B"]), C=t32(inp["C"]))
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        A_log, Dsk, dtb = t32(inp["A_log"]), t32(inp["D"]), t32(inp["dt_bias"])
        ys = [torch.empty_like(base["x"]) for _ in range(nsets)]

        calls = []
        for i, s in enumerate(sets):
            ops.ssm_scan_step(s["st"], s["x"], s["dr"], s["B"], s["C"], A_log, D_skip=Dsk, dt_bias=dtb, z=s["z"],
                              y=ys[i])
            calls.append(direct("ssm_scan_step", s["st"], s["x"], s["dr"], s["z"], s["B"], s["C"], A_log, Dsk, dtb,
                                ys[i], w.batch, w.dim, w.dstate, ops.SSM_F32, ops._stream()))

        def fn(i):
            calls[i]()

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f%% of 8 TB/s  sets=%d" %
            (name, ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, nsets))
        return dict(workload=w, bytes=nb, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs)

    def decode_case(name="step_b256_d5120", conv="conv_step_b256_d5120_k4"):
        # the fused decode step (conv1d step, then the scan step, one launch), and the
        # same token through the two separate launches for comparison
        w, cw = W.WORKLOADS[name], W.CONV_WORKLOADS[conv]
        inp, cin = W.make_inputs(w), W.make_conv_inputs(cw, batch=w.batch, dim=w.dim)
        nb = decode_bytes(w.batch, w.dim, w.dstate, cw.width, 4, w.gated)
        nsets = max(2, int(np.ceil(1.2e9 / nb)))
        base = dict(st=t32(inp["state"]), cs=t32(cin["state"]), x=t32(cin["x"]), dr=t32(inp["delta_raw"]),
                    z=t32(inp["z"]), B=t32(inp["B"]), C=t32(inp["C"]))
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        A_log, Dsk, dtb = t32(inp["A_log"]), t32(inp["D"]), t32(inp["dt_bias"])
        wt, cb = t32(cin["weight"]), t32(cin["bias"])
        ys = [torch.empty_like(base["x"]) for _ in range(nsets)]
        us = [torch.empty_like(base["x"]) for _ in range(nsets)]
        act = ops.SSM_ACT_SILU if cw.silu else ops.SSM_ACT_NONE
        fused, pair = [], []
        for i, s in enumerate(sets):
            ops.decode_step(s["cs"], s["x"], wt, s["st"], s["dr"], s["B"], s["C"], A_log, conv_bias=cb, silu=cw.silu,
                            D_skip=Dsk, dt_bias=dtb, z=s["z"], y=ys[i])
            fused.append(direct("ssm_decode_step", s["cs"], s["x"], wt, cb, cw.width, act, s["st"], s["dr"], s["z"],
                                s["B"], s["C"], A_log, Dsk, dtb, None, ys[i], w.batch, w.dim, w.dstate, ops.SSM_F32,
                                None, ops._stream()))
            c1 = direct("ssm_conv1d_step", s["cs"], s["x"], wt, cb, us[i], w.batch, w.dim, cw.width, act,
                        ops.SSM_F32, ops._stream())
            c2 = direct("ssm_scan_step", s["st"], us[i], s["dr"], s["z"], s["B"], s["C"], A_log, Dsk, dtb, ys[i],
                        w.batch, w.dim, w.dstate, ops.SSM_F32, ops._stream())
            pair.append((c1, c2))

        def fn(i):
            fused[i]()

        def fn_pair(i):
            pair[i][0]()
            pair[i][1]()

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        pw, pe, pm = timer.run(fn_pair, K, Wm, nsets)
        label = "decode_b%d_d%d_k%d" % (w.batch, w.dim, cw.width)
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f%% of 8 TB/s  sets=%d  "
            "(conv1d step + scan step as two launches: %.1f us)" %
            (label, ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, nsets, pe * 1e3))
        return dict(workload=w, bytes=nb, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs,
                    pair_us=pe * 1e3)

    def bwd_case(name="fwdbwd_b4_l2048_d2048", io="fp32", saved=False):
        # io = "bf16": the same workload with its activations, B, C and dy rounded to bf16
        # saved: the backward reuses chunk states written by the forward (made untimed)
        w = W.WORKLOADS[name]
        inp = W.make_inputs(w)
        b, l, d, n = w.batch, w.seqlen, w.dim, w.dstate
        nb = bwd_bytes(b, l, d, n, w.gated, 2 if io == "bf16" else 4)
        nsets = 2
        base = dict(x=tio(inp["x"], io), dr=tio(inp["delta_raw"], io), z=tio(inp["z"], io), B=tio(inp["B"], io),
                    C=tio(inp["C"], io), dy=tio(inp["dy"], io))
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        A_log, Dsk, dtb = t32(inp["A_log"]), t32(inp["D"]), t32(inp["dt_bias"])
        f = torch.float32
        a = torch.bfloat16 if io == "bf16" else f
        outs = [{"dx": torch.empty((b, l, d), dtype=a, device=dev), "ddelta_raw": torch.empty((b, l, d), dtype=a, device=dev),
                 "dz": torch.empty((b, l, d), dtype=a, device=dev), "dB": torch.empty((b, l, n), dtype=f, device=dev),
                 "dC": torch.empty((b, l, n), dtype=f, device=dev), "dA_log": torch.empty((d, n), dtype=f, device=dev),
                 "dD": torch.empty((d,), dtype=f, device=dev), "d_dt_bias": torch.empty((d,), dtype=f, device=dev)}
                for _ in range(nsets)]
        wsb = ops.bwd_workspace_bytes(b, l, d, n, ops.SSM_BF16 if io == "bf16" else ops.SSM_F32)
        wss = [torch.empty((wsb,), dtype=torch.uint8, device=dev) for _ in range(nsets)]
        css = [None] * nsets
        if saved:
            for i, s in enumerate(sets):
                css[i] = torch.empty(ops.chunk_states_shape(b, l, d, n), dtype=torch.float32, device=dev)
                ops.ssm_scan_fwd(s["x"], s["dr"], s["B"], s["C"], A_log, D_skip=Dsk, dt_bias=dtb, z=s["z"],
                                 return_final_state=False, chunk_states=css[i])
            torch.cuda.synchronize()

        def fn(i):
            s = sets[i]
            ops.ssm_scan_bwd(s["x"], s["dr"], s["B"], s["C"], A_log, s["dy"], D_skip=Dsk, dt_bias=dtb, z=s["z"],
                             workspace=wss[i], out=outs[i], chunk_states=css[i])

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        label = ("bwd_b4_l2048_d2048" if io == "fp32" else "bwd_bf16_b4_l2048_d2048") + ("_saved" if saved else "")
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f%% of 8 TB/s  workspace %.1f MB" %
            (label, ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, wsb / 1e6))
        return dict(workload=w, bytes=nb, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs, workspace_bytes=wsb)

    def mamba3_case(name="m3_b8_l2048_d2048"):
        w = W.MAMBA3_WORKLOADS[name]
        inp = W.make_mamba3_inputs(w)
        nb = mamba3_bytes(w.rows, w.inner, w.state, w.heads, w.rope_angles, w.bc_rows)
        nsets = 2
        g = inp["grads"]
        base = {"p": t32(inp["projected"]), **{k: t32(v) for k, v in g.items()}}
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        dtb = t32(inp["dt_bias"])
        outs = [(torch.empty_like(base["p"]), torch.empty((w.rows, w.heads), dtype=torch.float32, device=dev),
                 torch.empty((w.heads,), dtype=torch.float32, device=dev)) for _ in range(nsets)]

        def fn(i):
            s = sets[i]
            ops.mamba3_preprocess_bwd(s["p"], dtb, s["z"], s["x"], s["B"], s["C"], s["dt"], s["adt"], s["trap"],
                                      s["angles"], w.inner, w.state, w.heads, w.rope_angles, w.bc_rows, w.epsilon,
                                      w.dt_min, w.dt_max, w.a_floor, projected_grad=outs[i][0],
                                      dt_bias_partial=outs[i][1], d_dt_bias=outs[i][2])

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f%% of 8 TB/s  sets=%d" %
            (name, ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, nsets))
        return dict(workload=w, bytes=nb, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs)

    def ssd_case(name="ssd_b8_l2048_h64_w256", bwd=False):
        w = W.SSD_WORKLOADS[name]
        inp = W.make_ssd_inputs(w)
        nb = (ssd_bwd_bytes if bwd else ssd_fwd_bytes)(w.batch, w.seqlen, w.heads, w.nchunks, w.chunk)
        nsets = max(2, int(np.ceil(1.2e9 / nb)))
        keys = ("dt", "ddA", "ddt_out") if bwd else ("dt",)
        base = {k: t32(inp[k]) for k in keys}
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        A, dtb = t32(inp["A"]), t32(inp["dt_bias"])
        f = torch.float32
        if bwd:
            wsb = ops.ssd_chunk_cumsum_bwd_workspace_bytes(w.batch, w.seqlen, w.heads, w.chunk)
            outs = [{"ddt": torch.empty_like(base["dt"]), "dA": torch.empty((w.heads,), dtype=f, device=dev),
                     "db": torch.empty((w.heads,), dtype=f, device=dev),
                     "ws": torch.empty((wsb,), dtype=torch.uint8, device=dev)} for _ in range(nsets)]
        else:
            shp = (w.batch, w.heads, w.nchunks, w.chunk)
            outs = [{"cs": torch.empty(shp, dtype=f, device=dev), "dto": torch.empty(shp, dtype=f, device=dev)}
                    for _ in range(nsets)]

        calls = []
        sp = 1 if w.dt_softplus else 0
        for s, o in zip(sets, outs):
            if bwd:
                ops.ssd_chunk_cumsum_bwd(s["ddA"], s["ddt_out"], s["dt"], A, dt_bias=dtb, dt_softplus=w.dt_softplus,
                                         dt_min=w.dt_min, dt_max=w.dt_max, ddt=o["ddt"], workspace=o["ws"],
                                         dA=o["dA"], d_dt_bias=o["db"])
                calls.append(direct("ssm_ssd_chunk_cumsum_bwd", s["ddA"], s["ddt_out"], s["dt"], A, dtb, o["ddt"],
                                    o["dA"], o["db"], o["ws"], wsb, w.batch, w.seqlen, w.heads, w.chunk, sp,
                                    w.dt_min, w.dt_max, ops._stream()))
            else:
                ops.ssd_chunk_cumsum_fwd(s["dt"], A, w.chunk, dt_bias=dtb, dt_softplus=w.dt_softplus,
                                         dt_min=w.dt_min, dt_max=w.dt_max, dA_cumsum=o["cs"], dt_out=o["dto"])
                calls.append(direct("ssm_ssd_chunk_cumsum_fwd", s["dt"], A, dtb, o["cs"], o["dto"], w.batch,
                                    w.seqlen, w.heads, w.chunk, sp, w.dt_min, w.dt_max, ops._stream()))

        def fn(i):
            calls[i]()

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        label = ("ssd_cumsum_bwd_" if bwd else "ssd_cumsum_fwd_") + name[4:]
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f%% of 8 TB/s  sets=%d" %
            (label, ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, nsets))
        return dict(workload=w, bytes=nb, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs)

    def ssd_scan_case(name="ssd_scan_b8_l2048_h64_p64_n128"):
        w = W.SSD_SCAN_WORKLOADS[name]
        inp = W.make_ssd_scan_inputs(w)
        args = (w.batch, w.seqlen, w.heads, w.headdim, w.dstate, w.nchunks, w.chunk)
        nb, fl = ssd_scan_bytes(*args), ssd_scan_flops(*args)
        nsets = max(2, int(np.ceil(1.2e9 / nb)))
        A, dtb = t32(inp["A"]), t32(inp["dt_bias"])
        base = {k: t32(inp[k]) for k in ("x", "B", "C")}
        base["cs"], base["dto"] = ops.ssd_chunk_cumsum_fwd(t32(inp["dt"]), A, w.chunk, dt_bias=dtb)
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        Dv = t32(inp["D"])
        wsb = ops.ssd_chunk_scan_fwd_workspace_bytes(w.batch, w.seqlen, w.dstate)
        outs = [(torch.empty_like(base["x"]),
                 torch.empty((w.batch, w.heads, w.headdim, w.dstate), dtype=torch.float32, device=dev),
                 torch.empty((wsb,), dtype=torch.uint8, device=dev))
                for _ in range(nsets)]

        def fn(i):
            s = sets[i]
            ops.ssd_chunk_scan_fwd(s["x"], s["dto"], s["cs"], s["B"], s["C"], D=Dv, y=outs[i][0], h_final=outs[i][1],
                                   workspace=outs[i][2])

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        tfs = fl / (ev_ms * 1e-3) / 1e12
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f TFLOP/s = %.1f%% of fp32 MFMA 157.3  sets=%d"
            % (name, ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, tfs, 100 * tfs / 157.3, nsets))
        return dict(workload=w, bytes=nb, flops=fl, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs, tflops=tfs)

    def ssd_scan_bwd_case(name="ssd_scan_b8_l2048_h64_p64_n128"):
        w = W.SSD_SCAN_WORKLOADS[name]
        inp = W.make_ssd_scan_inputs(w)
        args = (w.batch, w.seqlen, w.heads, w.headdim, w.dstate, w.nchunks, w.chunk)
        nb, fl = ssd_scan_bwd_bytes(*args), ssd_scan_bwd_flops(*args)
        nsets = 2
        A, dtb, Dv = t32(inp["A"]), t32(inp["dt_bias"]), t32(inp["D"])
        dy = np.random.default_rng(w.seed).standard_normal(inp["x"].shape, dtype=np.float32)
        base = {k: t32(inp[k]) for k in ("x", "B", "C")}
        base["dy"] = t32(dy)
        base["cs"], base["dto"] = ops.ssd_chunk_cumsum_fwd(t32(inp["dt"]), A, w.chunk, dt_bias=dtb)
        base["bs"] = torch.empty(ops.ssd_block_states_shape(w.batch, w.seqlen, w.heads, w.headdim, w.dstate),
                                 dtype=torch.float32, device=dev)
        ops.ssd_chunk_scan_fwd(base["x"], base["dto"], base["cs"], base["B"], base["C"], D=Dv,
                               block_states=base["bs"])
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        wsb = ops.ssd_chunk_scan_bwd_workspace_bytes(w.batch, w.seqlen, w.heads, w.dstate)
        f = torch.float32
        outs = [{"dx": torch.empty_like(base["x"]), "ddA_cumsum": torch.empty_like(base["cs"]),
                 "ddt_out": torch.empty_like(base["dto"]),
                 "dB": torch.empty((w.batch, w.seqlen, w.dstate), dtype=f, device=dev),
                 "dC": torch.empty((w.batch, w.seqlen, w.dstate), dtype=f, device=dev),
                 "dD": torch.empty((w.heads,), dtype=f, device=dev),
                 "dh0": torch.empty((w.batch, w.heads, w.headdim, w.dstate), dtype=f, device=dev),
                 "ws": torch.empty((wsb,), dtype=torch.uint8, device=dev)} for _ in range(nsets)]

        def fn(i):
            s, o = sets[i], outs[i]
            ops.ssd_chunk_scan_bwd(s["x"], s["dto"], s["cs"], s["B"], s["C"], s["dy"], s["bs"], D=Dv,
                                   return_dh0=True, workspace=o["ws"], out={k: v for k, v in o.items() if k != "ws"})

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        tfs = fl / (ev_ms * 1e-3) / 1e12
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f TFLOP/s = %.1f%% of fp32 MFMA 157.3  "
            "workspace %.0f MB" % (name + "_bwd", ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, tfs, 100 * tfs / 157.3,
                                   wsb / 1e6))
        return dict(workload=w, bytes=nb, flops=fl, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs, tflops=tfs)

    def conv_case(name, min_bytes_rotation=1.2e9):
        w = W.CONV_WORKLOADS[name]
        inp = W.make_conv_inputs(w)
        es = 2 if w.io == "bf16" else 4
        step = w.kind == "conv_step"
        nb = conv_step_bytes(w.batch, w.dim, w.width, es) if step else conv_bytes(w.batch, w.seqlen, w.dim, w.width, es)
        nsets = max(2, int(np.ceil(min_bytes_rotation / nb)))
        base = {"x": tio(inp["x"], w.io)}
        if step:
            base["st"] = tio(inp["state"], w.io)
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        wt, bias = t32(inp["weight"]), t32(inp["bias"])
        outs = [torch.empty_like(base["x"]) for _ in range(nsets)]

        calls = []
        if step:
            io = ops.SSM_BF16 if w.io == "bf16" else ops.SSM_F32
            for i, s in enumerate(sets):
                ops.conv1d_step(s["st"], s["x"], wt, bias, silu=w.silu, out=outs[i])
                calls.append(direct("ssm_conv1d_step", s["st"], s["x"], wt, bias, outs[i], w.batch, w.dim, w.width,
                                    ops.SSM_ACT_SILU if w.silu else ops.SSM_ACT_NONE, io, ops._stream()))

        def fn(i):
            s = sets[i]
            if step:
                calls[i]()
            else:
                ops.conv1d_fwd(s["x"], wt, bias, silu=w.silu, out=outs[i])

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f%% of 8 TB/s  sets=%d" %
            (name, ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS, nsets))
        return dict(workload=w, bytes=nb, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs)

    def conv_bwd_case(name="conv_b8_l2048_d1536_k4"):
        w = W.CONV_WORKLOADS[name]
        inp = W.make_conv_inputs(w)
        nb = conv_bwd_bytes(w.batch, w.seqlen, w.dim, w.width)
        nsets = max(2, int(np.ceil(1.2e9 / nb)))
        base = {"x": t32(inp["x"]), "dout": t32(inp["dout"])}
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
        wt, bias = t32(inp["weight"]), t32(inp["bias"])
        f = torch.float32
        outs = [{"dx": torch.empty_like(base["x"]), "dw": torch.empty((w.dim, w.width), dtype=f, device=dev),
                 "db": torch.empty((w.dim,), dtype=f, device=dev)} for _ in range(nsets)]
        wsb = ops.conv1d_bwd_workspace_bytes(w.batch, w.seqlen, w.dim, w.width)
        wss = [torch.empty((wsb,), dtype=torch.uint8, device=dev) for _ in range(nsets)]

        def fn(i):
            s, o = sets[i], outs[i]
            ops.conv1d_bwd(s["x"], wt, s["dout"], bias, silu=w.silu, workspace=wss[i], dx=o["dx"], dweight=o["dw"],
                           dbias=o["db"])

        wall_ms, ev_ms, ev_min = timer.run(fn, K, Wm, nsets)
        gbs = nb / (ev_ms * 1e-3) / 1e9
        log("%-26s %8.1f us/launch (min %.1f, wall %.1f)  %7.1f GB/s  %.1f%% of 8 TB/s  sets=%d" %
            ("conv_bwd_b8_l2048_d1536_k4", ev_ms * 1e3, ev_min * 1e3, wall_ms * 1e3, gbs, 100 * gbs / HBM_PEAK_GBS,
             nsets))
        return dict(workload=w, bytes=nb, wall_ms=wall_ms, ev_ms=ev_ms, ev_min_ms=ev_min, gbs=gbs)

    if args.only == "copy":
        # calibration kernel for the HBM byte counters: a plain 1 GiB device-to-device copy
        nbytes = 1 << 30
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        bb = torch.empty_like(a)
        wall_ms, ev_ms, _ = timer.run(lambda i: bb.copy_(a), K, Wm, 1)
        log("copy 1 GiB: %.1f us, %.1f GB/s (read+write)" % (ev_ms * 1e3, 2 * nbytes / (ev_ms * 1e-3) / 1e9))
        print(json.dumps({"copy_bytes_each_way": nbytes, "ev_ms": ev_ms}))
        return

    head = None
    if args.only in ("all", "fwd"):
        head = fwd_case("fwd_b8_l2048_d1536")
    if args.only in ("all", "bf16"):
        results["fwd_bf16_b4_l4096_d4096"] = fwd_case("fwd_bf16_b4_l4096_d4096")
    if args.only in ("all", "fwd5"):
        results["fwd_b4_l2048_d2048"] = fwd_case("fwdbwd_b4_l2048_d2048")
    if args.only in ("all", "long"):
        results["fwd_long_b1_l65536_d1536"] = fwd_case("fwd_long_b1_l65536_d1536")
    if args.only in ("all", "step"):
        results["step_b256_d5120"] = step_case()
    if args.only in ("all", "decode"):
        results["decode_b256_d5120_k4"] = decode_case()
    if args.only in ("all", "bwd"):
        results["bwd_b4_l2048_d2048"] = bwd_case()
    if args.only in ("all", "bwd_bf16"):
        results["bwd_bf16_b4_l2048_d2048"] = bwd_case(io="bf16")
    if args.only in ("all", "train"):
        # the training pair with the forward's chunk states reused by the backward
        results["fwd_save_b4_l2048_d2048"] = fwd_case("fwdbwd_b4_l2048_d2048", save=True)
        results["bwd_saved_b4_l2048_d2048"] = bwd_case(saved=True)
    if args.only in ("all", "mamba3"):
        results["mamba3_preprocess_bwd_m3_b8_l2048_d2048"] = mamba3_case()
    if args.only in ("all", "ssd"):
        results["ssd_cumsum_fwd_b8_l2048_h64_w256"] = ssd_case()
        results["ssd_cumsum_bwd_b8_l2048_h64_w256"] = ssd_case(bwd=True)
        results["ssd_scan_fwd_b8_l2048_h64_p64_n128"] = ssd_scan_case()
        results["ssd_scan_bwd_b8_l2048_h64_p64_n128"] = ssd_scan_bwd_case()
    if args.only in ("all", "conv"):
        results["conv_b8_l2048_d1536_k4"] = conv_case("conv_b8_l2048_d1536_k4")
    if args.only in ("all", "conv_bf16"):
        results["conv_bf16_b4_l4096_d4096_k4"] = conv_case("conv_bf16_b4_l4096_d4096_k4")
    if args.only in ("all", "conv_step"):
        results["conv_step_b256_d5120_k4"] = conv_case("conv_step_b256_d5120_k4")
    if args.only in ("all", "conv_bwd"):
        results["conv_bwd_b8_l2048_d1536_k4"] = conv_bwd_case()

    if head is None:
        # profiling runs of a single secondary case print a short line
        print(json.dumps({k: {"gbs": v["gbs"], "us": v["ev_ms"] * 1e3} for k, v in results.items()}))
        return

    w = head["workload"]
    updates = w.state_updates
    valu_tslots = updates * SLOTS_PER_UPDATE / (head["ev_ms"] * 1e-3) / 1e12
    traffic = measured_traffic()
    roofline = {"bound": "hbm", "achieved": round(head["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(head["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": head["bytes"],
                "valu_issue_frac": round(valu_tslots / VALU_PEAK_TSLOTS, 4)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(head)
    secondary = {}
    for k, v in results.items():
        secondary[k] = {"gbs": round(v["gbs"], 1), "frac_of_8tbs": round(v["gbs"] / HBM_PEAK_GBS, 4),
                        "us_per_launch": round(v["ev_ms"] * 1e3, 1), "algorithmic_bytes": v["bytes"],
                        "elements_per_s": round(v["workload"].elements / (v["ev_ms"] * 1e-3), 1)}
        if "tflops" in v:
            secondary[k]["tflops"] = round(v["tflops"], 2)
            secondary[k]["frac_of_fp32_mfma"] = round(v["tflops"] / 157.3, 4)
            secondary[k]["flops"] = v["flops"]
        if v["workload"].kind in ("fwd", "fwdbwd"):
            secondary[k]["state_updates_per_s"] = round(v["workload"].state_updates / (v["ev_ms"] * 1e-3), 1)
        if "pair_us" in v:
            secondary[k]["two_launches_us"] = round(v["pair_us"], 1)

    out = {
        "metric": "selective-scan fwd achieved HBM GB/s and % of peak at 1 MI355X; step/bwd GB/s",
        "value": round(head["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(head["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fwd_b8_l2048_d1536", "batch": w.batch, "seqlen": w.seqlen, "d_inner": w.dim,
                   "d_state": w.dstate, "io": w.io, "gated": w.gated},
        "pct_of_hbm_peak": round(100 * head["gbs"] / HBM_PEAK_GBS, 2),
        "elements_per_s": round(w.elements / (head["ev_ms"] * 1e-3), 1),
        "state_updates_per_s": round(updates / (head["ev_ms"] * 1e-3), 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
