"""Compile the gfx950 HIP library libssmscan.so in-tree with hipcc.

Sources: csrc/ssm_api.hip (C ABI of include/ssm_scan.h and include/ssm_conv1d.h)
and the kernels in csrc/ssm_fwd.hip, csrc/ssm_step.hip, csrc/ssm_bwd.hip and
csrc/ssm_conv1d.hip, csrc/ssm_mamba3.hip and csrc/ssm_ssd.hip.  Each source is compiled separately (in parallel) and linked
into lib/libssmscan.so.  No fast-math; packed
fp32 instructions are disabled for the device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIBDIR, "libssmscan.so")
SOURCES = ["ssm_api.hip", "ssm_fwd.hip", "ssm_step.hip", "ssm_bwd.hip", "ssm_bwd_fused.hip", "ssm_conv1d.hip", "ssm_mamba3.hip", "ssm_ssd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libssmscan.so)")


def _flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I" + os.path.join(HERE, "..", "include")]


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        p = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
        if verbose and msgs.strip():
            print(msgs)
        return obj

    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
