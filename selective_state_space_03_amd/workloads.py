"""Named workloads and seeded synthetic inputs for the selective scan.

This module only draws random numbers and lays them out; it holds none of the
scan's arithmetic, so both the HIP path and the fp64 oracle can be fed from it.

Recipe (the same for every workload):
  * numpy ``Generator(PCG64(seed))``; draws are float64, rounded to float32
    (round-to-nearest-even) and, for bf16 I/O, further rounded to bf16 (RNE).
  * Fixed draw order: x, delta_raw, z, B, C, D_skip, u (for dt_bias), h0/state, dy.
  * x, delta_raw, z, B, C, dy ~ N(0, 1).  B and C are [batch, seqlen, dstate],
    i.e. shared by every channel of a (batch, time) position.
  * A_log[d, n] = log(n + 1), so A = -(n + 1) for every channel.
  * "bias" distributions:
      - "zero":  dt_bias = 0 and D_skip ~ N(0, 1)        (small fp32 case)
      - "mamba": dt_bias[d] = log(expm1(u_d)), u_d ~ U[1e-3, 1e-1] (so that
                 softplus(dt_bias) = u_d), and D_skip = 1.
  * A decode state (step workloads) ~ N(0, sd = 0.1).  Scans start from h0 = 0
    unless a test asks for a random h0 (also N(0, 0.1)).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str        # "fwd", "step" or "fwdbwd"
    batch: int
    seqlen: int
    dim: int         # d_inner, the channel count
    dstate: int      # N
    io: str          # "f32" or "bf16": dtype of x, delta_raw, z, B, C, y (state and params stay fp32)
    gated: bool
    bias: str        # "zero" or "mamba"
    seed: int

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.dim

    @property
    def state_updates(self) -> int:
        return self.elements * self.dstate


# The five workloads the build is measured and checked on, and the long-sequence one.
WORKLOADS = {
    "fwd_small": Workload("fwd_small", "fwd", 1, 64, 16, 4, "f32", False, "zero", 1001),
    "fwd_b8_l2048_d1536": Workload("fwd_b8_l2048_d1536", "fwd", 8, 2048, 1536, 16, "f32", True, "mamba", 1002),
    "fwd_bf16_b4_l4096_d4096": Workload("fwd_bf16_b4_l4096_d4096", "fwd", 4, 4096, 4096, 16, "bf16", True, "mamba", 1003),
    "step_b256_d5120": Workload("step_b256_d5120", "step", 256, 1, 5120, 16, "f32", True, "mamba", 1004),
    "fwdbwd_b4_l2048_d2048": Workload("fwdbwd_b4_l2048_d2048", "fwdbwd", 4, 2048, 2048, 16, "f32", True, "mamba", 1005),
    # one long sequence of few channels: the time-split forward
    "fwd_long_b1_l65536_d1536": Workload("fwd_long_b1_l65536_d1536", "fwd", 1, 65536, 1536, 16, "f32", True, "mamba",
                                         1006),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the raw uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_io(a: np.ndarray, io: str) -> np.ndarray:
    """float64 -> float32 (RNE) -> optionally bf16 (RNE); returned as float32 values."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    if io == "bf16":
        f = bf16_bits_to_f32(f32_to_bf16_bits(f))
    return f


def make_inputs(w: Workload, *, batch: Optional[int] = None, seqlen: Optional[int] = None,
                dim: Optional[int] = None, dstate: Optional[int] = None,
                gated: Optional[bool] = None, random_h0: bool = False,
                seed: Optional[int] = None, with_dy: Optional[bool] = None) -> dict:
    """Seeded inputs of workload ``w`` (optionally at other sizes, same distributions).

    Returns float32 numpy arrays (bf16-representable where ``w.io == "bf16"``):
      scan workloads: x, delta_raw, z|None, B, C, A_log, D, dt_bias, h0|None, dy|None
      step workloads: state, x, delta_raw, z|None, B, C, A_log, D, dt_bias
    plus "io" and the dims.
    """
    b = w.batch if batch is None else batch
    l = w.seqlen if seqlen is None else seqlen
    d = w.dim if dim is None else dim
    n = w.dstate if dstate is None else dstate
    g = w.gated if gated is None else gated
    want_dy = (w.kind == "fwdbwd") if with_dy is None else with_dy
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    io = w.io
    step = w.kind == "step"
    act = (b, d) if step else (b, l, d)
    bc = (b, n) if step else (b, l, n)

    x = round_to_io(rng.standard_normal(act), io)
    delta_raw = round_to_io(rng.standard_normal(act), io)
    z = round_to_io(rng.standard_normal(act), io) if g else None
    B = round_to_io(rng.standard_normal(bc), io)
    C = round_to_io(rng.standard_normal(bc), io)
    if w.bias == "zero":
        D = rng.standard_normal(d).astype(np.float32)
        dt_bias = np.zeros(d, np.float32)
    elif w.bias == "mamba":
        D = np.ones(d, np.float32)
        u = rng.uniform(1e-3, 1e-1, size=d)
        dt_bias = np.log(np.expm1(u)).astype(np.float32)
    else:
        raise ValueError("unknown bias distribution %r" % w.bias)
    A_log = np.broadcast_to(np.log(np.arange(1, n + 1, dtype=np.float64)), (d, n)).astype(np.float32)
    A_log = np.ascontiguousarray(A_log)
    out = {"io": io, "batch": b, "seqlen": 1 if step else l, "dim": d, "dstate": n,
           "x": x, "delta_raw": delta_raw, "z": z, "B": B, "C": C,
           "A_log": A_log, "D": D, "dt_bias": dt_bias}
    if step:
        out["state"] = (0.1 * rng.standard_normal((b, d, n))).astype(np.float32)
    else:
        out["h0"] = (0.1 * rng.standard_normal((b, d, n))).astype(np.float32) if random_h0 else None
        out["dy"] = round_to_io(rng.standard_normal((b, l, d)), io) if want_dy else None
    return out


# ---------------------------------------------------------------- depthwise causal conv1d
#
# The conv1d that precedes the scan in a Mamba block.  Recipe: numpy PCG64(seed); draw
# order x, w, bias, dout, state; x, dout, state ~ N(0, 1); w and bias ~ U(-1/sqrt(K),
# 1/sqrt(K)) (the default initialisation of a depthwise conv with K taps); values
# rounded to fp32 (and to bf16 for bf16 I/O) like the scan inputs.

@dataclasses.dataclass(frozen=True)
class ConvWorkload:
    name: str
    kind: str      # "conv" (sequence) or "conv_step" (one decode step)
    batch: int
    seqlen: int
    dim: int
    width: int     # K, taps per channel
    io: str
    silu: bool
    seed: int

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.dim


CONV_WORKLOADS = {
    "conv_small": ConvWorkload("conv_small", "conv", 1, 64, 16, 4, "f32", True, 2001),
    "conv_b8_l2048_d1536_k4": ConvWorkload("conv_b8_l2048_d1536_k4", "conv", 8, 2048, 1536, 4, "f32", True, 2002),
    "conv_bf16_b4_l4096_d4096_k4": ConvWorkload("conv_bf16_b4_l4096_d4096_k4", "conv", 4, 4096, 4096, 4, "bf16",
                                                True, 2003),
    "conv_step_b256_d5120_k4": ConvWorkload("conv_step_b256_d5120_k4", "conv_step", 256, 1, 5120, 4, "f32", True,
                                            2004),
}


def make_conv_inputs(w: ConvWorkload, *, batch: Optional[int] = None, seqlen: Optional[int] = None,
                     dim: Optional[int] = None, width: Optional[int] = None, silu: Optional[bool] = None,
                     seed: Optional[int] = None, io: Optional[str] = None) -> dict:
    """Seeded conv1d inputs: x ([b, l, d], or [b, d] for a step), weight [d, K], bias [d],
    dout like x, and for a step the state [b, d, K-1]."""
    b = w.batch if batch is None else batch
    l = w.seqlen if seqlen is None else seqlen
    d = w.dim if dim is None else dim
    k = w.width if width is None else width
    io_ = w.io if io is None else io
    step = w.kind == "conv_step"
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    act = (b, d) if step else (b, l, d)
    bound = 1.0 / np.sqrt(k)
    x = round_to_io(rng.standard_normal(act), io_)
    weight = rng.uniform(-bound, bound, size=(d, k)).astype(np.float32)
    bias = rng.uniform(-bound, bound, size=d).astype(np.float32)
    dout = rng.standard_normal(act).astype(np.float32)
    out = {"io": io_, "batch": b, "seqlen": 1 if step else l, "dim": d, "width": k,
           "silu": w.silu if silu is None else silu, "x": x, "weight": weight, "bias": bias, "dout": dout}
    if step:
        out["state"] = round_to_io(rng.standard_normal((b, d, k - 1)), io_)
    return out


# ---------------------------------------------------------- Mamba-3 preprocess adjoint

@dataclasses.dataclass(frozen=True)
class Mamba3Workload:
    """Adjoint of the Mamba-3 projection preprocess over `rows` token rows.  The page
    gives no sizes; these are a layer with d_model 2048 (inner 4096 = 64 heads of 64),
    state 128 in one B/C group and 64 rotary angles, over 8 x 2048 tokens."""
    name: str
    rows: int
    inner: int
    state: int
    heads: int
    rope_angles: int
    bc_rows: int
    epsilon: float = 1e-6
    dt_min: float = 1e-3
    dt_max: float = 1e-1
    a_floor: float = 1e-4
    seed: int = 2100

    @property
    def width(self):
        return 2 * self.inner + 2 * self.bc_rows * self.state + 3 * self.heads + self.rope_angles

    @property
    def kind(self):
        return "mamba3"

    @property
    def elements(self) -> int:  # elements of the gradient row written per launch
        return self.rows * self.width


MAMBA3_WORKLOADS = {
    "m3_small": Mamba3Workload("m3_small", rows=37, inner=70, state=16, heads=5, rope_angles=8, bc_rows=2, seed=2101),
    "m3_b8_l2048_d2048": Mamba3Workload("m3_b8_l2048_d2048", rows=8 * 2048, inner=4096, state=128, heads=64,
                                        rope_angles=64, bc_rows=1, seed=2102),
}


def make_mamba3_inputs(w: Mamba3Workload, *, rows: Optional[int] = None, inner: Optional[int] = None,
                       state: Optional[int] = None, heads: Optional[int] = None,
                       rope_angles: Optional[int] = None, bc_rows: Optional[int] = None,
                       seed: Optional[int] = None) -> dict:
    """Seeded fp32 inputs: projected rows ~ N(0, 1) (the dd_dt part shifted by the
    dt_bias draw as in the scan workloads), dt_bias = log(expm1(u)), u ~ U[1e-3, 1e-1],
    and every incoming gradient ~ N(0, 1).  Draw order: projected, u, z, x, B, C, dt,
    adt, trap, angles gradients."""
    r = w.rows if rows is None else rows
    inn = w.inner if inner is None else inner
    st = w.state if state is None else state
    hd = w.heads if heads is None else heads
    ang = w.rope_angles if rope_angles is None else rope_angles
    bc = w.bc_rows if bc_rows is None else bc_rows
    width = 2 * inn + 2 * bc * st + 3 * hd + ang
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    f = np.float32
    projected = rng.standard_normal((r, width)).astype(f)
    u = rng.uniform(1e-3, 1e-1, hd)
    dt_bias = np.log(np.expm1(u)).astype(f)
    g = {k: rng.standard_normal((r, n)).astype(f) for k, n in
         (("z", inn), ("x", inn), ("B", bc * st), ("C", bc * st), ("dt", hd), ("adt", hd), ("trap", hd),
          ("angles", ang))}
    return {"rows": r, "inner": inn, "state": st, "heads": hd, "rope_angles": ang, "bc_rows": bc,
            "epsilon": w.epsilon, "dt_min": w.dt_min, "dt_max": w.dt_max, "a_floor": w.a_floor,
            "projected": projected, "dt_bias": dt_bias, "grads": g}


# ---------------------------------------------------------------- Mamba-2 SSD chunk cumsum

@dataclasses.dataclass(frozen=True)
class SsdWorkload:
    """Chunk cumsum of the Mamba-2 SSD scan over [batch, seqlen, heads] step sizes.  The
    page gives no sizes; the large one is a layer with d_model 2048 (64 heads of 64
    channels) over 8 x 2048 tokens with 256-step chunks."""
    name: str
    batch: int
    seqlen: int
    heads: int
    chunk: int
    dt_softplus: bool = True
    dt_min: float = 0.0
    dt_max: float = float("inf")
    seed: int = 2200

    @property
    def kind(self):
        return "ssd"

    @property
    def nchunks(self) -> int:
        return (self.seqlen + self.chunk - 1) // self.chunk

    @property
    def elements(self) -> int:  # step sizes per launch
        return self.batch * self.seqlen * self.heads


SSD_WORKLOADS = {
    "ssd_small": SsdWorkload("ssd_small", batch=2, seqlen=300, heads=20, chunk=64, seed=2201),
    "ssd_b8_l2048_h64_w256": SsdWorkload("ssd_b8_l2048_h64_w256", batch=8, seqlen=2048, heads=64, chunk=256,
                                         seed=2202),
}


def make_ssd_inputs(w: SsdWorkload, *, batch: Optional[int] = None, seqlen: Optional[int] = None,
                    heads: Optional[int] = None, chunk: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """Seeded fp32 inputs of the chunk cumsum and its backward: dt ~ N(0, 1) (raw step
    sizes before the bias), u ~ U[1e-3, 1e-1] with dt_bias = log(expm1(u)), A = -u'
    with u' ~ U[1, 16] (Mamba-2's initial decay rates), and the incoming chunk
    gradients ddA, ddt_out ~ N(0, 1).  Draw order: dt, u, u', ddA, ddt_out."""
    b = w.batch if batch is None else batch
    l = w.seqlen if seqlen is None else seqlen
    h = w.heads if heads is None else heads
    W = w.chunk if chunk is None else chunk
    nc = (l + W - 1) // W
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    f = np.float32
    dt = rng.standard_normal((b, l, h)).astype(f)
    u = rng.uniform(1e-3, 1e-1, h)
    dt_bias = np.log(np.expm1(u)).astype(f)
    A = (-rng.uniform(1.0, 16.0, h)).astype(f)
    ddA = rng.standard_normal((b, h, nc, W)).astype(f)
    ddt_out = rng.standard_normal((b, h, nc, W)).astype(f)
    return {"batch": b, "seqlen": l, "heads": h, "chunk": W, "dt": dt, "dt_bias": dt_bias, "A": A, "ddA": ddA,
            "ddt_out": ddt_out}


@dataclasses.dataclass(frozen=True)
class SsdScanWorkload:
    """SSD scan forward over [batch, seqlen, heads, headdim] inputs with one B/C group of
    d_state, in chunks of `chunk` steps.  The page gives no sizes: a d_model-2048 Mamba-2
    layer (64 heads of 64 channels, d_state 128) over 8 x 2048 tokens."""
    name: str
    batch: int
    seqlen: int
    heads: int
    headdim: int
    dstate: int
    chunk: int = 64
    seed: int = 2300

    @property
    def kind(self):
        return "ssd_scan"

    @property
    def nchunks(self) -> int:
        return (self.seqlen + self.chunk - 1) // self.chunk

    @property
    def elements(self) -> int:  # outputs y per launch
        return self.batch * self.seqlen * self.heads * self.headdim


SSD_SCAN_WORKLOADS = {
    "ssd_scan_small": SsdScanWorkload("ssd_scan_small", batch=2, seqlen=150, heads=3, headdim=64, dstate=128, seed=2301),
    "ssd_scan_b8_l2048_h64_p64_n128": SsdScanWorkload("ssd_scan_b8_l2048_h64_p64_n128", batch=8, seqlen=2048,
                                                      heads=64, headdim=64, dstate=128, seed=2302),
}


def make_ssd_scan_inputs(w: SsdScanWorkload, *, batch: Optional[int] = None, seqlen: Optional[int] = None,
                         heads: Optional[int] = None, dstate: Optional[int] = None, h0: bool = False,
                         seed: Optional[int] = None) -> dict:
    """Seeded fp32 inputs: x ~ N(0, 1) [batch, seqlen, heads, headdim], raw dt ~ N(0, 1)
    [batch, seqlen, heads], u ~ U[1e-3, 1e-1] with dt_bias = log(expm1(u)), A = -U[1, 16],
    B, C ~ N(0, 1) [batch, seqlen, dstate], D = 1, and (when asked) h0 ~ N(0, 1).  Draw
    order: x, dt, u, A, B, C, h0."""
    b = w.batch if batch is None else batch
    l = w.seqlen if seqlen is None else seqlen
    h = w.heads if heads is None else heads
    n = w.dstate if dstate is None else dstate
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    f = np.float32
    x = rng.standard_normal((b, l, h, w.headdim), dtype=np.float32)
    dt = rng.standard_normal((b, l, h)).astype(f)
    u = rng.uniform(1e-3, 1e-1, h)
    dt_bias = np.log(np.expm1(u)).astype(f)
    A = (-rng.uniform(1.0, 16.0, h)).astype(f)
    Bm = rng.standard_normal((b, l, n)).astype(f)
    Cm = rng.standard_normal((b, l, n)).astype(f)
    h0v = rng.standard_normal((b, h, w.headdim, n)).astype(f) if h0 else None
    return {"batch": b, "seqlen": l, "heads": h, "headdim": w.headdim, "dstate": n, "chunk": w.chunk, "x": x,
            "dt": dt, "dt_bias": dt_bias, "A": A, "B": Bm, "C": Cm, "D": np.ones(h, f), "h0": h0v}
