"""Build the gfx950 shared library ``libparo.so`` in-tree with hipcc.

Usage: ``python -m rotated_w4_linear_amd.build`` (or ``build()`` from Python).
Each source is compiled to an object of its own (in parallel, under
``_build/``), then the objects are linked; every call recompiles everything.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libparo.so")

SOURCES = ["api.cpp", "plan.cpp", "pairs.cpp", "rotate.hip", "quantize.hip", "w4_linear.hip", "decode.hip",
           "backward.hip", "layer_loss.hip", "noalloc.hip", "dense_gemm.hip", "measure.hip"]

COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                         # every rounding is explicit (fma builtins where wanted)
    "-fhip-fp32-correctly-rounded-divide-sqrt",  # IEEE division in the quantizer
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
LINK_FLAGS = [
    "--offload-arch=gfx950", "-shared", "-fPIC",
    "-Wl,-z,defs",                                # no undefined symbols (e.g. a kernel stub) in the library
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _quiet(stderr: str) -> str:
    # the host pass does not know the packed-fp32 target feature: harmless
    return "\n".join(ln for ln in (stderr or "").splitlines() if "packed-fp32-ops" not in ln)


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMPILE_FLAGS, "-I", os.path.join(HERE, "..", "include"), *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} ({res.returncode}):\n{_quiet(res.stderr)}")
    if verbose and _quiet(res.stderr).strip():
        print(_quiet(res.stderr), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libparo.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as pool:
        objs = list(pool.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *LINK_FLAGS, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_quiet(res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
