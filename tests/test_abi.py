"""CPU checks of the C ABI: the library loads, exports every function that
include/*.h declares, and rejects invalid arguments with the documented
status codes *before* enqueueing anything.  Every call here fails validation, so
no HIP call is made and no GPU is needed (pointer values are fake addresses that
are never dereferenced)."""
import ctypes
import os
import re

import pytest
import torch

from selective_state_space_03_amd import ops

# Every call below is built to fail validation.  As a second line of defence, the
# fake-pointer calls never run where a GPU is visible: a call that passed
# validation by mistake would launch a kernel on addresses that do not exist.
no_gpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                 reason="fake-pointer validation checks run only where no GPU is visible")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, NULL, DIM, UNSUP, ALIGN, WS, ALIAS = 0, 1, 2, 3, 4, 5, 6


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(ssm_\w+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(ops.EXPORTS), names
    L = ops.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = ops.lib()
    for code, name in ops.STATUS.items():
        assert L.ssm_status_string(code).decode().startswith(name)
    assert b"unknown" in L.ssm_status_string(99)


# fake, well-aligned, non-overlapping device addresses (never dereferenced)
BASE = 1 << 40
STRIDE = 1 << 32


def addr(i, off=0):
    return ctypes.c_void_p(BASE + i * STRIDE + off)


def fwd_args(**over):
    a = dict(x=addr(0), delta_raw=addr(1), z=addr(2), B=addr(3), C=addr(4), A_log=addr(5), D=addr(6),
             dt_bias=addr(7), h0=None, y=addr(8), h_final=addr(9), b=2, l=16, d=64, n=16,
             io=ops.SSM_F32, ws=None, wsb=0, stream=None)
    a.update(over)
    return a


def call_fwd(a):
    return ops.lib().ssm_scan_fwd(a["x"], a["delta_raw"], a["z"], a["B"], a["C"], a["A_log"], a["D"],
                                  a["dt_bias"], a["h0"], a["y"], a["h_final"], a["b"], a["l"], a["d"],
                                  a["n"], a["io"], a["ws"], a["wsb"], a["stream"])


@no_gpu_only
@pytest.mark.parametrize("field", ["x", "delta_raw", "B", "C", "A_log", "y"])
def test_fwd_null_required_pointer(field):
    assert call_fwd(fwd_args(**{field: None})) == NULL


@no_gpu_only
@pytest.mark.parametrize("over", [dict(n=0), dict(n=17), dict(b=0), dict(l=0), dict(d=0), dict(l=-5),
                                  dict(b=1 << 40, l=1 << 20)])
def test_fwd_bad_dims(over):
    assert call_fwd(fwd_args(**over)) == DIM


@no_gpu_only
def test_fwd_bad_dtype():
    assert call_fwd(fwd_args(io=7)) == UNSUP


@no_gpu_only
def test_fwd_misaligned():
    assert call_fwd(fwd_args(x=addr(0, 2))) == ALIGN            # fp32 needs 4 B
    assert call_fwd(fwd_args(y=addr(8, 1), io=ops.SSM_BF16)) == ALIGN
    assert call_fwd(fwd_args(A_log=addr(5, 2))) == ALIGN
    assert call_fwd(fwd_args(B=addr(3, 2))) == ALIGN            # fp32 B needs 4 B


@no_gpu_only
def test_fwd_aliasing():
    assert call_fwd(fwd_args(y=addr(0))) == ALIAS               # y == x
    assert call_fwd(fwd_args(h_final=addr(5))) == ALIAS         # h_final == A_log
    assert call_fwd(fwd_args(h_final=addr(8, 64))) == ALIAS     # inside y


def test_workspace_sizes():
    L = ops.lib()
    assert L.ssm_scan_fwd_workspace_bytes(8, 2048, 1536, 16, 0) == 0
    wb = L.ssm_scan_bwd_workspace_bytes(4, 2048, 2048, 16, 0)
    assert wb > 0 and wb % 256 == 0
    assert L.ssm_scan_bwd_workspace_bytes(4, 2048, 2048, 17, 0) == 0   # invalid sizes
    # grows with every size
    assert L.ssm_scan_bwd_workspace_bytes(4, 4096, 2048, 16, 0) > wb
    assert L.ssm_scan_bwd_workspace_bytes(8, 2048, 2048, 16, 0) > wb


def step_call(**over):
    a = dict(state=addr(0), x=addr(1), delta_raw=addr(2), z=addr(3), B=addr(4), C=addr(5), A_log=addr(6),
             D=addr(7), dt_bias=addr(8), y=addr(9), b=4, d=64, n=16, io=ops.SSM_F32, stream=None)
    a.update(over)
    return ops.lib().ssm_scan_step(a["state"], a["x"], a["delta_raw"], a["z"], a["B"], a["C"], a["A_log"],
                                   a["D"], a["dt_bias"], a["y"], a["b"], a["d"], a["n"], a["io"], a["stream"])


@no_gpu_only
def test_step_validation():
    assert step_call(state=None) == NULL
    assert step_call(y=None) == NULL
    assert step_call(n=0) == DIM
    assert step_call(n=20) == DIM
    assert step_call(io=2) == UNSUP
    assert step_call(state=addr(0, 2)) == ALIGN
    assert step_call(y=addr(1)) == ALIAS      # y == x
    assert step_call(state=addr(6)) == ALIAS  # state == A_log


def bwd_call(**over):
    a = dict(x=addr(0), delta_raw=addr(1), z=addr(2), B=addr(3), C=addr(4), A_log=addr(5), D=addr(6),
             dt_bias=addr(7), h0=None, dy=addr(8), dx=addr(9), ddelta_raw=addr(10), dz=addr(11), dB=addr(12),
             dC=addr(13), dA_log=addr(14), dD=addr(15), d_dt_bias=addr(16), ws=addr(17), wsb=None,
             b=2, l=64, d=128, n=16, io=ops.SSM_F32, stream=None)
    a.update(over)
    if a["wsb"] is None:
        a["wsb"] = ops.lib().ssm_scan_bwd_workspace_bytes(a["b"], a["l"], a["d"], min(max(a["n"], 1), 16), 0)
    return ops.lib().ssm_scan_bwd(a["x"], a["delta_raw"], a["z"], a["B"], a["C"], a["A_log"], a["D"],
                                  a["dt_bias"], a["h0"], a["dy"], a["dx"], a["ddelta_raw"], a["dz"], a["dB"],
                                  a["dC"], a["dA_log"], a["dD"], a["d_dt_bias"], a["ws"], a["wsb"], a["b"],
                                  a["l"], a["d"], a["n"], a["io"], a["stream"])


@no_gpu_only
def test_bwd_validation():
    assert bwd_call(dy=None) == NULL
    assert bwd_call(dz=None) == NULL                 # z given, dz missing
    assert bwd_call(dB=None) == NULL
    assert bwd_call(n=0) == DIM
    assert bwd_call(io=7) == UNSUP
    assert bwd_call(io=ops.SSM_BF16, dy=addr(8, 1)) == ALIGN   # bf16 needs 2 B
    assert bwd_call(io=ops.SSM_BF16, dB=addr(12, 2)) == ALIGN  # dB stays fp32
    assert bwd_call(ws=None) == WS
    assert bwd_call(wsb=1024) == WS
    assert bwd_call(ws=addr(17, 64)) == WS           # workspace must be 256 B aligned
    assert bwd_call(dx=addr(0)) == ALIAS             # dx == x
    assert bwd_call(ws=addr(9)) == ALIAS             # workspace == dx
    assert bwd_call(dB=addr(13)) == ALIAS            # dB == dC
    assert bwd_call(dA_log=addr(14, 2)) == ALIGN



def decode_call(**over):
    a = dict(cs=addr(10), x=addr(1), w=addr(11), cb=addr(12), k=4, act=1, state=addr(0), delta_raw=addr(2),
             z=addr(3), B=addr(4), C=addr(5), A_log=addr(6), D=addr(7), dt_bias=addr(8), u=addr(13), y=addr(9),
             b=4, d=64, n=16, io=ops.SSM_F32, opts=None, stream=None)
    a.update(over)
    return ops.lib().ssm_decode_step(a["cs"], a["x"], a["w"], a["cb"], a["k"], a["act"], a["state"],
                                     a["delta_raw"], a["z"], a["B"], a["C"], a["A_log"], a["D"], a["dt_bias"],
                                     a["u"], a["y"], a["b"], a["d"], a["n"], a["io"], a["opts"], a["stream"])


@no_gpu_only
def test_decode_step_validation():
    assert decode_call(state=None) == NULL
    assert decode_call(w=None) == NULL
    assert decode_call(cs=None) == NULL              # width 4 needs the conv state
    assert decode_call(n=0) == DIM
    assert decode_call(k=0) == DIM
    assert decode_call(k=9) == DIM
    assert decode_call(io=2) == UNSUP
    assert decode_call(act=5) == UNSUP
    assert decode_call(cs=addr(10, 2)) == ALIGN       # fp32 conv state needs 4 B
    assert decode_call(io=ops.SSM_BF16, u=addr(13, 1)) == ALIGN
    assert decode_call(w=addr(11, 2)) == ALIGN
    assert decode_call(y=addr(1)) == ALIAS           # y == x
    assert decode_call(u=addr(9)) == ALIAS           # u == y
    assert decode_call(cs=addr(11)) == ALIAS         # conv state == weight
    assert decode_call(cs=addr(0, 64)) == ALIAS      # conv state inside the scan state
    o = ops.ScanOptions(dt_min=0.5, dt_max=0.1)
    assert decode_call(opts=ctypes.pointer(o)) == 8  # SSM_ERR_ARG: dt_min > dt_max

# ---------------------------------------------------------------- conv1d

def conv_call(x=addr(0), w=addr(5), bias=addr(6), out=addr(9), b=2, l=64, d=32, k=4, act=1, io=0):
    return ops.lib().ssm_conv1d_fwd(x, w, bias, out, b, l, d, k, act, io, None)


@no_gpu_only
def test_conv_fwd_validation():
    assert conv_call(x=None) == NULL
    assert conv_call(w=None) == NULL
    assert conv_call(k=0) == DIM and conv_call(k=9) == DIM and conv_call(l=0) == DIM
    assert conv_call(act=2) == UNSUP and conv_call(io=5) == UNSUP
    assert conv_call(x=addr(0, 2)) == ALIGN
    assert conv_call(out=addr(0)) == ALIAS


@no_gpu_only
def test_conv_step_and_bwd_validation():
    L = ops.lib()
    # step: a width > 1 needs a state; in-place state may not overlap x
    assert L.ssm_conv1d_step(None, addr(0), addr(5), None, addr(9), 2, 32, 4, 1, 0, None) == NULL
    assert L.ssm_conv1d_step(addr(0), addr(0), addr(5), None, addr(9), 2, 32, 4, 1, 0, None) == ALIAS
    # bwd: fp32 only, and the workspace is required and large enough
    wsb = L.ssm_conv1d_bwd_workspace_bytes(2, 64, 32, 4, 0)
    assert wsb > 0
    assert L.ssm_conv1d_bwd(addr(0), addr(5), None, addr(1), addr(9), None, None, addr(11), wsb, 2, 64, 32, 4, 1,
                            1, None) == UNSUP
    assert L.ssm_conv1d_bwd(addr(0), addr(5), None, addr(1), addr(9), None, None, None, wsb, 2, 64, 32, 4, 1, 0,
                            None) == WS
    assert L.ssm_conv1d_bwd(addr(0), addr(5), None, addr(1), addr(9), None, None, addr(11), wsb - 1, 2, 64, 32, 4,
                            1, 0, None) == WS
    assert L.ssm_conv1d_bwd(addr(0), addr(5), None, addr(1), addr(0), None, None, addr(11), wsb, 2, 64, 32, 4, 1,
                            0, None) == ALIAS


@no_gpu_only
def test_conv_bwd_noalloc_validation():
    """The no-allocation backward checks like ssm_conv1d_bwd, and refuses sizes whose
    workspace exceeds its fixed scratch with SSM_ERR_SCRATCH, before any HIP call."""
    L = ops.lib()
    SCRATCH = 9
    assert L.ssm_conv1d_bwd_noalloc(None, addr(5), None, addr(1), addr(9), None, None, 2, 64, 32, 4, 1, 0,
                                    None) == NULL
    assert L.ssm_conv1d_bwd_noalloc(addr(0), addr(5), None, addr(1), addr(9), None, None, 2, 64, 32, 4, 1, 1,
                                    None) == UNSUP
    assert L.ssm_conv1d_bwd_noalloc(addr(0), addr(5), None, addr(1), addr(0), None, None, 2, 64, 32, 4, 1, 0,
                                    None) == ALIAS
    # many short sequences: one partial per batch element, 128 MB of partials
    big = (100000, 16, 64, 4)
    assert L.ssm_conv1d_bwd_workspace_bytes(*big, 0) > ops.CONV1D_SCRATCH_BYTES
    assert L.ssm_conv1d_bwd_noalloc(addr(0), addr(5), None, addr(1), addr(9), None, None, *big, 1, 0,
                                    None) == SCRATCH
    # the benchmark's conv shape fits
    assert L.ssm_conv1d_bwd_workspace_bytes(8, 2048, 1536, 4, 0) <= ops.CONV1D_SCRATCH_BYTES


# ------------------------------------------------ options of the _ex entry points

def _opts(dt_min=0.0, dt_max=0.0, dh_final=None, dh0=None):
    return ctypes.pointer(ops.ScanOptions(dt_min, dt_max, dh_final, dh0))


ARG = 8


def call_fwd_ex(a, opts):
    return ops.lib().ssm_scan_fwd_ex(a["x"], a["delta_raw"], a["z"], a["B"], a["C"], a["A_log"], a["D"],
                                     a["dt_bias"], a["h0"], a["y"], a["h_final"], a["b"], a["l"], a["d"],
                                     a["n"], a["io"], a["ws"], a["wsb"], opts, a["stream"])


def bwd_ex_call(opts, **over):
    a = dict(x=addr(0), delta_raw=addr(1), z=addr(2), B=addr(3), C=addr(4), A_log=addr(5), D=addr(6),
             dt_bias=addr(7), h0=None, dy=addr(8), dx=addr(9), ddelta_raw=addr(10), dz=addr(11), dB=addr(12),
             dC=addr(13), dA_log=addr(14), dD=addr(15), d_dt_bias=addr(16), ws=addr(17), b=2, l=64, d=128, n=16)
    a.update(over)
    wsb = ops.lib().ssm_scan_bwd_workspace_bytes(a["b"], a["l"], a["d"], a["n"], 0)
    return ops.lib().ssm_scan_bwd_ex(a["x"], a["delta_raw"], a["z"], a["B"], a["C"], a["A_log"], a["D"],
                                     a["dt_bias"], a["h0"], a["dy"], a["dx"], a["ddelta_raw"], a["dz"], a["dB"],
                                     a["dC"], a["dA_log"], a["dD"], a["d_dt_bias"], a["ws"], wsb, a["b"],
                                     a["l"], a["d"], a["n"], ops.SSM_F32, opts, None)


@no_gpu_only
def test_options_validation():
    a = fwd_args()
    nan = float("nan")
    assert call_fwd_ex(a, _opts(0.2, 0.1)) == ARG            # dt_min > dt_max
    assert call_fwd_ex(a, _opts(-0.1, 1.0)) == ARG           # negative lower bound
    assert call_fwd_ex(a, _opts(nan, 1.0)) == ARG
    assert call_fwd_ex(a, _opts(0.0, nan)) == ARG
    assert call_fwd_ex(a, _opts(dh_final=BASE + 20 * STRIDE)) == ARG   # backward-only field
    assert call_fwd_ex(a, _opts(dh0=BASE + 20 * STRIDE)) == ARG
    assert call_fwd_ex(fwd_args(x=None), _opts(0.2, 0.1)) == NULL  # pointer checks come first
    L = ops.lib()
    st = L.ssm_scan_step_ex(addr(0), addr(1), addr(2), addr(3), addr(4), addr(5), addr(6), addr(7), addr(8),
                            addr(9), 4, 64, 16, ops.SSM_F32, _opts(1.0, 0.5), None)
    assert st == ARG
    # backward: the state gradients are validated like every other buffer
    assert bwd_ex_call(_opts(0.3, 0.2)) == ARG
    assert bwd_ex_call(_opts(dh0=BASE + 0 * STRIDE)) == ALIAS            # dh0 == x
    assert bwd_ex_call(_opts(dh0=BASE + 9 * STRIDE)) == ALIAS            # dh0 == dx
    assert bwd_ex_call(_opts(dh_final=BASE + 9 * STRIDE)) == ALIAS       # dh_final == dx
    assert bwd_ex_call(_opts(dh0=BASE + 20 * STRIDE + 2)) == ALIGN
    assert bwd_ex_call(_opts(dh_final=BASE + 20 * STRIDE + 1)) == ALIGN


@no_gpu_only
def test_chunk_states_validation():
    L = ops.lib()
    assert L.ssm_scan_chunk_states_bytes(2, 33, 64, 16) == 2 * 3 * 16 * 64 * 4   # ceil(33/16) chunks
    assert L.ssm_scan_chunk_states_bytes(2, 33, 64, 17) == 0
    cs = BASE + 20 * STRIDE

    def opt(p):
        o = ops.ScanOptions(0.0, 0.0, None, None, p)
        return ctypes.pointer(o)

    assert call_fwd_ex(fwd_args(n=8), opt(cs)) == UNSUP            # saved by the d_state 9..16 kernel only
    assert call_fwd_ex(fwd_args(), opt(BASE + 8 * STRIDE)) == ALIAS  # chunk states == y
    assert call_fwd_ex(fwd_args(), opt(BASE + 0 * STRIDE)) == ALIAS  # chunk states == x
    assert call_fwd_ex(fwd_args(), opt(cs + 2)) == ALIGN
    assert call_fwd_ex(fwd_args(b=1, l=1 << 20, d=1024), opt(cs)) == UNSUP  # one batch element's part >= 2^31 B
    st = L.ssm_scan_step_ex(addr(0), addr(1), addr(2), addr(3), addr(4), addr(5), addr(6), addr(7), addr(8),
                            addr(9), 4, 64, 16, ops.SSM_F32, opt(cs), None)
    assert st == ARG                                                  # not a step option
    assert bwd_ex_call(opt(BASE + 9 * STRIDE)) == ALIAS              # chunk states == dx
    assert bwd_ex_call(opt(cs + 1)) == ALIGN


@no_gpu_only
def test_mamba3_validation():
    L = ops.lib()

    def call(rows=4, inner=8, state=4, heads=2, angles=2, bc=1, eps=1e-6, lo=1e-3, hi=0.1, floor=1e-4, **over):
        p = dict(projected=addr(0), dt_bias=addr(1), zg=addr(2), xg=addr(3), bg=addr(4), cg=addr(5), dtg=addr(6),
                 adtg=addr(7), trapg=addr(8), angg=addr(9), out=addr(10), part=addr(11), dbias=addr(12))
        p.update(over)
        ws = p.get("ws", addr(13))
        wsb = p.get("wsb", L.ssm_mamba3_preprocess_bwd_workspace_bytes(rows, heads))
        return L.ssm_mamba3_preprocess_bwd(p["projected"], p["dt_bias"], p["zg"], p["xg"], p["bg"], p["cg"],
                                           p["dtg"], p["adtg"], p["trapg"], p["angg"], p["out"], p["part"],
                                           p["dbias"], ws, wsb, rows, inner, state, heads, angles, bc, eps, lo, hi,
                                           floor, None)
    assert call(rows=0) == DIM and call(inner=-1) == DIM and call(state=0) == DIM
    assert call(projected=None) == NULL and call(out=None) == NULL and call(part=None) == NULL
    assert call(angg=None) == NULL
    assert call(eps=-1.0) == ARG and call(lo=0.2, hi=0.1) == ARG and call(lo=-1.0) == ARG
    assert call(floor=float("nan")) == ARG
    assert call(out=addr(0)) == ALIAS and call(part=addr(10)) == ALIAS and call(dbias=addr(1)) == ALIAS
    assert call(out=addr(10, 2)) == ALIGN
    assert call(ws=None) == WS and call(wsb=16) == WS and call(ws=addr(13, 64)) == WS
    assert call(ws=addr(10)) == ALIAS                    # workspace == projected_grad
    assert L.ssm_mamba3_preprocess_bwd_workspace_bytes(130, 64) == 768            # 3 chunks x 64 heads x 4 B
    assert L.ssm_mamba3_preprocess_bwd_workspace_bytes(130, 3) == 256             # rounded up to 256 B


@no_gpu_only
def test_ssd_chunk_cumsum_validation():
    L = ops.lib()
    inf = float("inf")

    def fwd(b=2, l=100, h=8, w=64, sp=1, lo=0.0, hi=inf, **over):
        p = dict(dt=addr(0), A=addr(1), bias=addr(2), cs=addr(3), dto=addr(4))
        p.update(over)
        return L.ssm_ssd_chunk_cumsum_fwd(p["dt"], p["A"], p["bias"], p["cs"], p["dto"], b, l, h, w, sp, lo, hi,
                                          None)

    def bwd(b=2, l=100, h=8, w=64, sp=1, lo=0.0, hi=inf, **over):
        p = dict(ddA=addr(0), ddo=addr(1), dt=addr(2), A=addr(3), bias=addr(4), ddt=addr(5), dA=addr(6),
                 db=addr(7), ws=addr(8))
        p.update(over)
        wsb = p.get("wsb", L.ssm_ssd_chunk_cumsum_bwd_workspace_bytes(b, l, h, w))
        return L.ssm_ssd_chunk_cumsum_bwd(p["ddA"], p["ddo"], p["dt"], p["A"], p["bias"], p["ddt"], p["dA"],
                                          p["db"], p["ws"], wsb, b, l, h, w, sp, lo, hi, None)
    for f in (fwd, bwd):
        assert f(b=0) == DIM and f(l=0) == DIM and f(h=0) == DIM and f(w=0) == DIM
        assert f(h=(1 << 20) + 1) == DIM and f(b=1 << 16, l=1 << 16) == DIM
        assert f(lo=-1.0) == ARG and f(lo=0.5, hi=0.1) == ARG and f(hi=float("nan")) == ARG
        assert f(A=None) == NULL and f(dt=None) == NULL
    assert fwd(cs=None) == NULL and fwd(dto=None) == NULL
    assert fwd(cs=addr(0)) == ALIAS and fwd(dto=addr(3)) == ALIAS and fwd(cs=addr(2)) == ALIAS
    assert fwd(cs=addr(3, 2)) == ALIGN
    assert bwd(ddA=None) == NULL and bwd(ddt=None) == NULL and bwd(dA=None) == NULL
    assert bwd(ws=None) == WS and bwd(wsb=16) == WS and bwd(ws=addr(8, 64)) == WS
    assert bwd(ddt=addr(2)) == ALIAS and bwd(ws=addr(5)) == ALIAS and bwd(db=addr(6)) == ALIAS
    assert bwd(ddt=addr(5, 1)) == ALIGN
    # two [batch, chunks, heads] fp32 partial arrays, each rounded up to 256 bytes
    assert L.ssm_ssd_chunk_cumsum_bwd_workspace_bytes(2, 100, 8, 64) == 2 * 256
    assert L.ssm_ssd_chunk_cumsum_bwd_workspace_bytes(8, 2048, 64, 256) == 2 * 8 * 8 * 64 * 4
    assert L.ssm_ssd_chunk_cumsum_bwd_workspace_bytes(0, 100, 8, 64) == 0


@no_gpu_only
def test_ssd_chunk_scan_validation():
    L = ops.lib()

    def call(b=2, l=100, h=3, p=64, n=128, w=64, **over):
        a = dict(x=addr(0), dto=addr(1), cs=addr(2), B=addr(3), C=addr(4), D=addr(5), h0=addr(6), y=addr(7),
                 hf=addr(8), bs=addr(9), ws=addr(10))
        a.update(over)
        wsb = a.get("wsb", L.ssm_ssd_chunk_scan_fwd_workspace_bytes(b, l, n))
        return L.ssm_ssd_chunk_scan_fwd(a["x"], a["dto"], a["cs"], a["B"], a["C"], a["D"], a["h0"], a["y"], a["hf"],
                                        a["bs"], a["ws"], wsb, b, l, h, p, n, w, None)
    assert call(b=0) == DIM and call(l=0) == DIM and call(p=0) == DIM and call(w=0) == DIM
    assert call(p=32) == UNSUP and call(n=96) == UNSUP and call(w=96) == UNSUP and call(w=32) == UNSUP
    assert call(x=None) == NULL and call(cs=None) == NULL and call(y=None) == NULL
    assert call(y=addr(0)) == ALIAS and call(hf=addr(6)) == ALIAS and call(hf=addr(7)) == ALIAS
    assert call(y=addr(7, 2)) == ALIGN and call(bs=addr(9, 2)) == ALIGN
    assert call(bs=addr(0)) == ALIAS and call(bs=addr(8)) == ALIAS
    assert call(ws=None) == WS and call(wsb=16) == WS and call(ws=addr(10, 64)) == WS
    assert call(ws=addr(3)) == ALIAS and call(ws=addr(7)) == ALIAS
    # C_i.B_s of every 64-step block: [batch, blocks, 64, 64] fp32 (2 x 2 x 16 KB)
    assert L.ssm_ssd_chunk_scan_fwd_workspace_bytes(2, 100, 128) == 2 * 2 * 64 * 64 * 4
    assert L.ssm_ssd_chunk_scan_fwd_workspace_bytes(0, 100, 128) == 0


@no_gpu_only
def test_ssd_chunk_scan_bwd_validation():
    L = ops.lib()

    def call(b=2, l=100, h=3, p=64, n=128, w=64, **over):
        a = dict(x=addr(0), dto=addr(1), cs=addr(2), B=addr(3), C=addr(4), D=addr(5), dy=addr(6), bs=addr(7),
                 dhf=addr(8), dx=addr(9), dcs=addr(10), ddt=addr(11), dB=addr(12), dC=addr(13), dD=addr(14),
                 dh0=addr(15), ws=addr(16))
        a.update(over)
        wsb = a.get("wsb", L.ssm_ssd_chunk_scan_bwd_workspace_bytes(b, l, h, n))
        return L.ssm_ssd_chunk_scan_bwd(a["x"], a["dto"], a["cs"], a["B"], a["C"], a["D"], a["dy"], a["bs"], a["dhf"],
                                        a["dx"], a["dcs"], a["ddt"], a["dB"], a["dC"], a["dD"], a["dh0"], a["ws"], wsb,
                                        b, l, h, p, n, w, None)
    assert call(b=0) == DIM and call(l=0) == DIM and call(n=0) == DIM
    assert call(p=32) == UNSUP and call(n=96) == UNSUP and call(w=128) == UNSUP
    assert call(bs=None) == NULL and call(dy=None) == NULL and call(dB=None) == NULL and call(ddt=None) == NULL
    assert call(dx=addr(0)) == ALIAS and call(dB=addr(13)) == ALIAS and call(ws=addr(9)) == ALIAS
    assert call(dx=addr(9, 2)) == ALIGN
    assert call(ws=None) == WS and call(wsb=16) == WS and call(ws=addr(16, 64)) == WS
    # G of every (batch, head, 64-step chunk), [64, N] fp32; dD per (batch, chunk, head);
    # with at most 128 (batch, chunk) pairs the heads are split into groups (here 3
    # groups of 1) and each group's dB and dC ([batch, seqlen, N] fp32) is kept
    assert L.ssm_ssd_chunk_scan_bwd_workspace_bytes(2, 100, 3, 128) == 2 * 3 * 2 * 64 * 128 * 4 + 256 + 2 * 307200
    # 256 (batch, chunk) pairs: one group, dB and dC written in place
    assert L.ssm_ssd_chunk_scan_bwd_workspace_bytes(8, 2048, 64, 128) == 8 * 64 * 32 * 64 * 128 * 4 + 8 * 32 * 64 * 4
