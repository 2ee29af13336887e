"""Shared helpers of the GPU tests: device placement of seeded inputs, the error
metric, and a flushed progress line before each GPU step."""
import sys

import numpy as np

RTOL_F32 = 1e-4   # max relative error bound for fp32 I/O
RTOL_BF16 = 2e-2  # ... for bf16 I/O with an fp32 state


def say(msg):
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def rel_err(g, r):
    """max_i |g_i - r_i| / max(|r_i|, rms(r)): relative error with the tensor's RMS as
    the floor, so that values crossing zero do not make the ratio meaningless."""
    g = np.asarray(g, dtype=np.float64).ravel()
    r = np.asarray(r, dtype=np.float64).ravel()
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    floor = rms if rms > 0 else 1.0
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))


def tol(io):
    return RTOL_BF16 if io == "bf16" else RTOL_F32


def to_dev(a, io, device="cuda"):
    """float32 numpy (bf16-representable when io == bf16) -> device tensor of the io dtype."""
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if io == "bf16" else t


def to_dev32(a, device="cuda"):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t):
    return t.detach().float().cpu().numpy()
