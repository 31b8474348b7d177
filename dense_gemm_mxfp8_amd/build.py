"""Build the HIP library ``libgemm.so`` in-tree for gfx950 with hipcc.

Each source is compiled to an object under ``_build/`` (the GEMM kernels and
the attention kernel are separate translation units), then the objects are
linked into one shared library.  ``build()`` always compiles every source;
``build(only=[...])`` recompiles just the named sources and relinks with the
existing objects of the others.

``build(measure=True)`` (``python -m dense_gemm_mxfp8_amd.build --measure``)
makes a second library, ``libgemm_measure.so``, compiled with
``-DLIBGEMM_MEASURE``: in it the ``LIBGEMM_*`` environment switches that force
a kernel variant are live (the product library has none).  ``bench.py
--measure-build`` loads it; nothing else does.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "libgemm.hip"), os.path.join(PKG, "csrc", "gemm_mf16.hip"),
           os.path.join(PKG, "csrc", "attention.hip")]
# Per-source flags: the 16 x 16 MFMA kernel is compiled without the machine
# scheduler that runs before register allocation (its reordering of the 64
# accumulator quads of a wave tile made the allocator move accumulators around
# the MFMAs); the kernel fixes its instruction interleave itself.
SOURCE_FLAGS = {"gemm_mf16.hip": ["-mllvm", "-enable-misched=0"]}
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgemm.so")
MEASURE_LIBRARY = os.path.join(PKG, "libgemm_measure.so")
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


def _object(src: str, measure: bool = False) -> str:
    d = os.path.join(BUILD_DIR, "measure") if measure else BUILD_DIR
    return os.path.join(d, os.path.splitext(os.path.basename(src))[0] + ".o")


def build(verbose: bool = False, only=None, measure: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(os.path.dirname(_object(SOURCES[0], measure)), exist_ok=True)
    defines = ["-DLIBGEMM_MEASURE"] if measure else []
    todo = SOURCES if only is None else [s for s in SOURCES if os.path.basename(s) in only]

    def compile_one(src):
        obj = _object(src, measure)
        extra = SOURCE_FLAGS.get(os.path.basename(src), [])
        _run([hipcc, *HIPCC_FLAGS, *extra, *defines, f"-I{INCLUDE}", "-c", src, "-o", obj + ".tmp"], verbose)
        os.replace(obj + ".tmp", obj)

    # the translation units compile independently (each hipcc is one process)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(len(todo), os.cpu_count() or 1))) as pool:
        for f in [pool.submit(compile_one, src) for src in todo]:
            f.result()
    out = MEASURE_LIBRARY if measure else LIBRARY
    tmp = out + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[_object(s, measure) for s in SOURCES], "-o", tmp],
         verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    args = [a for a in sys.argv[1:] if a != "--measure"]
    print(build(verbose=True, only=args or None, measure="--measure" in sys.argv[1:]))
