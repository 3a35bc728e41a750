"""Routed int4 Mixture-of-Experts layer for AMD MI355X (gfx950).

The compute lives in libqmoe.so (HIP, C ABI in include/qmoe.h); this package is the thin
Python binding over it.  Build the library with ``python -m quantized_moe_router_amd.build``.
"""
from ._lib import QmoeError, lib, make_dims, EXPORTS, LIB_PATH  # noqa: F401
from . import ops  # noqa: F401

__all__ = ["QmoeError", "lib", "make_dims", "EXPORTS", "LIB_PATH", "ops"]
