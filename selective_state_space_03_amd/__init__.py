"""MI355X-native (gfx950) Mamba selective-scan hot path.

The compute runs in hand-written HIP kernels inside ``libssmscan.so`` behind a
C ABI (``include/ssm_scan.h``); ``selective_state_space_03_amd.ops`` is the thin
Python binding over it.  ``workloads`` holds the named workloads and seeded
synthetic inputs.  Importing this package loads nothing: the library is loaded
on first use of the binding and its absence is an error, never a fallback.
"""
__all__ = ["ops", "workloads"]
