"""Per-rank compute of a Megatron-style column->row tensor-parallel block on one MI355X (gfx950).

The product is the C ABI in include/tpshard.h, implemented by libtpshard.so (HIP kernels in csrc/).  This package
holds the build step, the ctypes binding (same names as the C ABI) and a small rank-loop driver that allocates
buffers with torch and calls the ABI.  Nothing here falls back to another implementation: without the built
library every entry point raises.
"""
from __future__ import annotations

from .build import LIB_PATH, build, is_current  # noqa: F401

_BINDING = None


def load():
    """The ctypes binding module.  Builds the library first when there is no built copy, or when the copy was built
    from other sources or flags than the ones in the tree (a hash recorded at build time), so a stale binary is
    never used."""
    global _BINDING
    if _BINDING is None:
        if not is_current():
            build()
        from . import _lib

        _BINDING = _lib
    return _BINDING


def __getattr__(name):
    if name.startswith("tp_") or name in ("TpError", "make_dims", "tp_dims", "lib"):
        return getattr(load(), name)
    raise AttributeError(name)
