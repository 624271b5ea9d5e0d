"""MI355X-native fused causal differential attention (and Grouped Differential
Attention): hand-written gfx950 HIP kernels behind a C ABI (libdiffattn.so),
with a thin Python binding.  PyTorch supplies device memory and streams only.

The shared library is loaded on first use; every op raises if it is missing.
"""
from .workloads import WORKLOADS, ORDER  # noqa: F401

__all__ = ["WORKLOADS", "ORDER"]
