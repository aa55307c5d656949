"""Build libeagle.so in-tree with hipcc for gfx950.

    python -m eagle_draft_tree_expand_amd.build      # or build() from Python

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel)
and linked into lib/libeagle.so.  Packed-fp32 instruction selection is
disabled for all device code.  build(debug=True) makes lib/libeagle_debug.so
(objects in _build_debug/): the same code with EAGLE_LDS_CHECK, whose tree
assembly and acceptance walk check their LDS indices (EAGLE_STATUS_LDS_INDEX).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
BUILD_DEBUG = os.path.join(PKG, "_build_debug")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libeagle.so")
LIB_DEBUG = os.path.join(LIBDIR, "libeagle_debug.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source and link the shared library (the debug library
    with debug=True); returns its path."""
    bdir, lib = (BUILD_DEBUG, LIB_DEBUG) if debug else (BUILD, LIB)
    flags = FLAGS + (["-DEAGLE_LDS_CHECK"] if debug else [])
    os.makedirs(bdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    hipcc = _hipcc()
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        cmd = [hipcc, *flags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = r.stdout + r.stderr
        # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, debug="--debug" in sys.argv[1:]))
