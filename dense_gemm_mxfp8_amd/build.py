"""Build the HIP library ``libgemm.so`` in-tree for gfx950 with hipcc.

Each source is compiled to an object under ``_build/`` (the GEMM kernels and
the attention kernel are separate translation units), then the objects are
linked into one shared library.  ``build()`` always compiles every source;
``build(only=[...])`` recompiles just the named sources and relinks with the
existing objects of the others.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "libgemm.hip"), os.path.join(PKG, "csrc", "attention.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgemm.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")


def _object(src: str) -> str:
    return os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")


def build(verbose: bool = False, only=None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    todo = SOURCES if only is None else [s for s in SOURCES if os.path.basename(s) in only]
    for src in todo:
        obj = _object(src)
        _run([hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", "-c", src, "-o", obj + ".tmp"], verbose)
        os.replace(obj + ".tmp", obj)
    tmp = LIBRARY + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[_object(s) for s in SOURCES], "-o", tmp],
         verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    import sys
    print(build(verbose=True, only=sys.argv[1:] or None))
