"""Build the HIP library ``libsq.so`` in-tree for gfx950.

Run ``python w8a8_int8_quantization_amd/build.py`` (or ``__graft_entry__.build()``); this
file imports nothing from the package, whose import needs the built library.
Every build compiles from source; nothing is cached outside this directory.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsq.so")
ARCH = "gfx950"

# -ffp-contract=off: every binary32 multiply and add rounds on its own, as the
# method's definitions are written; fused multiply-adds appear only where a
# kernel asks for one.  Packed FP32 instructions are disabled.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build_library(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + [f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
