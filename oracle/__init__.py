"""fp64 CPU oracle of the Mamba selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and the oracle shares no code
with that path: the arithmetic lives in ``ssm_oracle.c`` (plain C, built with
gcc, no GPU headers), this module only marshals numpy arrays.

Every input is widened to float64 before the call: fp32 inputs widen exactly,
and bf16 inputs are passed as the float values they represent (also exact).

Functions (definitions and citations are in the headers of ``ssm_oracle.c`` and
``conv1d_oracle.c``):
  fwd(...)  -> {"y", "h_final"}          forward scan, sequential in t
  step(...) -> {"y", "state"}            single decode step (separate code)
  bwd(...)  -> {"dx", "ddelta_raw", "dz", "dB", "dC", "dA_log", "dD", "d_dt_bias", "dh0"}
  (fwd, step and bwd take the step-size clamp dt_min, dt_max; bwd takes dh_final)
  softplus / sigmoid / silu / silu_grad  scalar helpers, exposed for pinning
  conv_fwd(...)  -> out                  depthwise causal conv1d (+ SiLU)
  conv_step(...) -> {"out", "state"}     one decode step of it (separate code)
  conv_bwd(...)  -> {"dx", "dw", "dbias"}
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "ssm_oracle.c"), os.path.join(_HERE, "conv1d_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "libssm_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile the oracle's C sources with gcc into libssm_oracle.so (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-shared", "-fPIC",
               "-std=c99", "-D_POSIX_C_SOURCE=200809L"] + _SRCS + ["-o", tmp, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        L = ctypes.c_long
        Dbl = ctypes.c_double
        lib.ssm_oracle_fwd.argtypes = [P] * 11 + [L] * 4 + [Dbl, Dbl, ctypes.c_int]
        lib.ssm_oracle_fwd.restype = ctypes.c_int
        lib.ssm_oracle_step.argtypes = [P] * 10 + [L] * 3 + [Dbl, Dbl, ctypes.c_int]
        lib.ssm_oracle_step.restype = ctypes.c_int
        lib.ssm_oracle_bwd.argtypes = [P] * 20 + [L] * 4 + [Dbl, Dbl, ctypes.c_int]
        lib.ssm_oracle_bwd.restype = ctypes.c_int
        lib.conv1d_oracle_fwd.argtypes = [P] * 4 + [L] * 4 + [ctypes.c_int]
        lib.conv1d_oracle_fwd.restype = ctypes.c_int
        lib.conv1d_oracle_step.argtypes = [P] * 5 + [L] * 3 + [ctypes.c_int]
        lib.conv1d_oracle_step.restype = ctypes.c_int
        lib.conv1d_oracle_bwd.argtypes = [P] * 7 + [L] * 4 + [ctypes.c_int]
        lib.conv1d_oracle_bwd.restype = ctypes.c_int
        for name in ("softplus", "sigmoid", "silu", "silu_grad"):
            f = getattr(lib, "ssm_oracle_" + name)
            f.argtypes = [ctypes.c_double]
            f.restype = ctypes.c_double
        _lib = lib
        return lib


def default_threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(x, delta_raw, B, C, A_log, D=None, dt_bias=None, z=None, h0=None, nthreads=None,
        dt_min=0.0, dt_max=float("inf")):
    x = _f64(x)
    b, l, d = x.shape
    n = np.asarray(A_log).shape[1]
    delta_raw = _f64(delta_raw, (b, l, d))
    z = _f64(z, (b, l, d))
    B = _f64(B, (b, l, n))
    C = _f64(C, (b, l, n))
    A_log = _f64(A_log, (d, n))
    D = _f64(D, (d,))
    dt_bias = _f64(dt_bias, (d,))
    h0 = _f64(h0, (b, d, n))
    y = np.empty((b, l, d), np.float64)
    h_final = np.empty((b, d, n), np.float64)
    rc = _load().ssm_oracle_fwd(_ptr(x), _ptr(delta_raw), _ptr(z), _ptr(B), _ptr(C), _ptr(A_log),
                                _ptr(D), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(h_final),
                                b, l, d, n, float(dt_min), float(dt_max), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("ssm_oracle_fwd failed with %d" % rc)
    return {"y": y, "h_final": h_final}


def step(state, x, delta_raw, B, C, A_log, D=None, dt_bias=None, z=None, nthreads=None,
         dt_min=0.0, dt_max=float("inf")):
    state = np.array(state, dtype=np.float64, copy=True, order="C")
    b, d, n = state.shape
    x = _f64(x, (b, d))
    delta_raw = _f64(delta_raw, (b, d))
    z = _f64(z, (b, d))
    B = _f64(B, (b, n))
    C = _f64(C, (b, n))
    A_log = _f64(A_log, (d, n))
    D = _f64(D, (d,))
    dt_bias = _f64(dt_bias, (d,))
    y = np.empty((b, d), np.float64)
    rc = _load().ssm_oracle_step(_ptr(state), _ptr(x), _ptr(delta_raw), _ptr(z), _ptr(B), _ptr(C),
                                 _ptr(A_log), _ptr(D), _ptr(dt_bias), _ptr(y), b, d, n,
                                 float(dt_min), float(dt_max), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("ssm_oracle_step failed with %d" % rc)
    return {"y": y, "state": state}


def bwd(x, delta_raw, B, C, A_log, dy, D=None, dt_bias=None, z=None, h0=None, nthreads=None,
        dt_min=0.0, dt_max=float("inf"), dh_final=None):
    x = _f64(x)
    b, l, d = x.shape
    n = np.asarray(A_log).shape[1]
    delta_raw = _f64(delta_raw, (b, l, d))
    z = _f64(z, (b, l, d))
    B = _f64(B, (b, l, n))
    C = _f64(C, (b, l, n))
    A_log = _f64(A_log, (d, n))
    D = _f64(D, (d,))
    dt_bias = _f64(dt_bias, (d,))
    h0 = _f64(h0, (b, d, n))
    dy = _f64(dy, (b, l, d))
    dh_final = _f64(dh_final, (b, d, n))
    out = {
        "dx": np.empty((b, l, d)), "ddelta_raw": np.empty((b, l, d)),
        "dz": np.empty((b, l, d)) if z is not None else None,
        "dB": np.empty((b, l, n)), "dC": np.empty((b, l, n)),
        "dA_log": np.empty((d, n)), "dD": np.empty((d,)), "d_dt_bias": np.empty((d,)),
        "dh0": np.empty((b, d, n)),
    }
    rc = _load().ssm_oracle_bwd(
        _ptr(x), _ptr(delta_raw), _ptr(z), _ptr(B), _ptr(C), _ptr(A_log), _ptr(D), _ptr(dt_bias),
        _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(out["dx"]), _ptr(out["ddelta_raw"]), _ptr(out["dz"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dA_log"]), _ptr(out["dD"]),
        _ptr(out["d_dt_bias"]), _ptr(out["dh0"]), b, l, d, n, float(dt_min), float(dt_max),
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("ssm_oracle_bwd failed with %d" % rc)
    return out


def softplus(r: float) -> float:
    return _load().ssm_oracle_softplus(float(r))


def sigmoid(r: float) -> float:
    return _load().ssm_oracle_sigmoid(float(r))


def silu(z: float) -> float:
    return _load().ssm_oracle_silu(float(z))


def silu_grad(z: float) -> float:
    return _load().ssm_oracle_silu_grad(float(z))


# ---------------------------------------------------------------- conv1d

def conv_fwd(x, w, bias=None, silu=True):
    x = _f64(x)
    b, l, d = x.shape
    w = _f64(w)
    k = w.shape[1]
    w = _f64(w, (d, k))
    bias = _f64(bias, (d,))
    out = np.empty((b, l, d), np.float64)
    rc = _load().conv1d_oracle_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(out), b, l, d, k, int(bool(silu)))
    if rc != 0:
        raise RuntimeError("conv1d_oracle_fwd failed with %d" % rc)
    return out


def conv_step(state, x, w, bias=None, silu=True):
    x = _f64(x)
    b, d = x.shape
    w = _f64(w)
    k = w.shape[1]
    w = _f64(w, (d, k))
    bias = _f64(bias, (d,))
    state = np.array(state, dtype=np.float64, copy=True, order="C").reshape(b, d, k - 1)
    out = np.empty((b, d), np.float64)
    rc = _load().conv1d_oracle_step(_ptr(state) if k > 1 else None, _ptr(x), _ptr(w), _ptr(bias), _ptr(out),
                                    b, d, k, int(bool(silu)))
    if rc != 0:
        raise RuntimeError("conv1d_oracle_step failed with %d" % rc)
    return {"out": out, "state": state}


def conv_bwd(x, w, dout, bias=None, silu=True):
    x = _f64(x)
    b, l, d = x.shape
    w = _f64(w)
    k = w.shape[1]
    w = _f64(w, (d, k))
    bias = _f64(bias, (d,))
    dout = _f64(dout, (b, l, d))
    out = {"dx": np.empty((b, l, d)), "dw": np.empty((d, k)), "dbias": np.empty((d,))}
    rc = _load().conv1d_oracle_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(dout), _ptr(out["dx"]), _ptr(out["dw"]),
                                   _ptr(out["dbias"]), b, l, d, k, int(bool(silu)))
    if rc != 0:
        raise RuntimeError("conv1d_oracle_bwd failed with %d" % rc)
    return out
