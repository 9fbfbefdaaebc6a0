"""Per-rank compute of a Megatron-style column->row tensor-parallel block on one MI355X (gfx950).

The product is the C ABI in include/tpshard.h, implemented by libtpshard.so (HIP kernels in csrc/).  This package
holds the build step, the ctypes binding (same names as the C ABI) and a small rank-loop driver that allocates
buffers with torch and calls the ABI.  Nothing here falls back to another implementation: without the built
library every entry point raises.
"""
from __future__ import annotations

import os

from .build import LIB_PATH, build  # noqa: F401

_BINDING = None


def load():
    """The ctypes binding module; builds the library first if no built copy exists."""
    global _BINDING
    if _BINDING is None:
        if not os.path.exists(LIB_PATH):
            build()
        from . import _lib

        _BINDING = _lib
    return _BINDING


def __getattr__(name):
    if name.startswith("tp_") or name in ("TpError", "make_dims", "tp_dims", "lib"):
        return getattr(load(), name)
    raise AttributeError(name)
