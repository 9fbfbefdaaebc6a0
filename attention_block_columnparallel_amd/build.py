"""Build libtpshard.so in-tree with hipcc for gfx950.

Each HIP source compiles to an object under _build/ (in parallel), then one link step makes the shared object
next to this file.  Run as `python -m attention_block_columnparallel_amd.build` or call build().
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libtpshard.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# sha256 of the sources and flags a library was built from, written next to it by build()
HASH_PATH = LIB_PATH + ".srchash"
ARCH = "gfx950"

SOURCES = ["tp_abi.hip", "comm_kernels.hip", "gemm_bf16.hip", "gemm_f32.hip", "attention.hip", "sp_region.hip", "vocab_ce.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-I" + INCLUDE,
    "-I" + CSRC,
    # keep the compiler from forming packed fp32 vector ops by itself
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def source_hash(extra_flags=()) -> str:
    """sha256 over every file under csrc/, the C header, the source list and the compile flags (include paths
    relative to the repository, so a copy of the tree at another path hashes the same)."""
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if not f.startswith("."))
    for path in files + [os.path.join(INCLUDE, "tpshard.h")]:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
    flags = [f.replace(ROOT, "<root>") for f in COMMON_FLAGS + list(extra_flags)]
    h.update("\0".join(SOURCES + flags).encode())
    return h.hexdigest()


def built_hash() -> str:
    """The source hash recorded by the build that made the current library ("" if none)."""
    try:
        with open(HASH_PATH) as fh:
            return fh.read().strip()
    except OSError:
        return ""


def is_current() -> bool:
    """True when the built library exists and was built from the sources and flags as they are now."""
    return os.path.exists(LIB_PATH) and built_hash() == source_hash()


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(hipcc: str, src: str, obj: str, extra) -> None:
    cmd = [hipcc, *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source for gfx950 and link libtpshard.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = []
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, hipcc, src, obj, list(extra_flags)))
        for f in futs:
            f.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    with open(HASH_PATH + ".tmp", "w") as fh:
        fh.write(source_hash(extra_flags) + "\n")
    os.replace(HASH_PATH + ".tmp", HASH_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
