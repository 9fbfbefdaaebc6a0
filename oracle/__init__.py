"""Oracle package: the fp64 CPU reference for the tensor-parallel block.

TEST INFRASTRUCTURE ONLY: imported by the tests, __graft_entry__.smoke() and bench.py's CPU-baseline leg, never by
the library.  Parity status: every function is pinned by the CPU tests; none is "parity unpinned".
"""
from .tp_oracle import *  # noqa: F401,F403
from . import tp_oracle  # noqa: F401
