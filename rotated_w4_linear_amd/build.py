"""Build the gfx950 shared library ``libparo.so`` in-tree with hipcc.

Usage: ``python -m rotated_w4_linear_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libparo.so")

SOURCES = ["api.cpp", "plan.cpp", "rotate.hip", "quantize.hip", "w4_linear.hip", "decode.hip",
           "backward.hip", "layer_loss.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                         # every rounding is explicit (fma builtins where wanted)
    "-fhip-fp32-correctly-rounded-divide-sqrt",  # IEEE division in the quantizer
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-Wl,-z,defs",                                # no undefined symbols (e.g. a kernel stub) in the library
    "-L/opt/rocm/lib", "-lrocblas",               # the layer loss's dense products
    "-Wl,-rpath,/opt/rocm/lib",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source into libparo.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(HERE, "..", "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in (res.stderr or "").splitlines()
                    if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
