"""MI355X-native routed-token scatter -> grouped GEMM MoE expert path.

The computation lives in libmoe.so (HIP kernels for gfx950 behind the C ABI of
include/moe.h); ``_lib`` binds it with ctypes and ``layer.MoELayer`` chains the
calls.  ``inputs`` draws the seeded synthetic workloads.
"""
from . import _lib  # noqa: F401
from .layer import MoELayer  # noqa: F401

__all__ = ["MoELayer"]
