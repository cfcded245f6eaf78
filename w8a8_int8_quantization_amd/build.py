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
# measurement probes for the benchmark's probe modes (not part of the layer)
PROBE_SRC = os.path.join(PKG, "probes", "probes.hip")
PROBE_LIB = os.path.join(PKG, "libsq_probes.so")
ARCH = "gfx950"

# -ffp-contract=off: every binary32 multiply and add rounds on its own, as the
# method's definitions are written; fused multiply-adds appear only where a
# kernel asks for one.  Packed FP32 instructions are disabled.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Extra objects built from a source with other flags: the E4M3 host code of
# the prefill GEMM (gemm_big.hip with SQ_BIG_E4M3), compiled without LLVM's
# machine-code sinking, which otherwise moves the E4M3 main loop's matrix
# instructions past the conditional stage transfers of the hand-over substep,
# so a stage's twelve MFMAs issue back to back after all of its fragment reads
# (QKV prefill E4M3 GEMM 59.2 -> 48.4 us without the pass; the int8 instances
# are compiled as before).
EXTRA_OBJECTS = [("gemm_big.hip", "gemm_big.e4m3.o", ["-DSQ_BIG_E4M3", "-mllvm", "-disable-machine-sink"])]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, obj: str, extra=()) -> str:
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + ["-c", f"-I{INCLUDE}", f"-I{CSRC}", "-o", obj, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({res.returncode}):\n{out}")
    return out


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (libsq_san.so, for the CPU tests of the C-ABI layer): each
# -fsanitize= applies to the host compilation only (-Xarch_host), the gfx950
# device code is built as usual.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(PKG, "libsq_san.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that a host process must preload to load libsq_san.so."""
    clang = os.path.join(os.path.dirname(hipcc()), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def build_library(verbose: bool = False, jobs: int = 0, sanitize: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libsq.so
    (libsq_san.so with sanitize=True)."""
    from concurrent.futures import ThreadPoolExecutor

    srcs = sources()
    objdir = os.path.join(PKG, "_build_san" if sanitize else "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = SAN_FLAGS if sanitize else []
    units = [(s, os.path.join(objdir, os.path.basename(s) + ".o"), extra) for s in srcs]
    units += [(os.path.join(CSRC, src), os.path.join(objdir, obj), flags + extra) for src, obj, flags in EXTRA_OBJECTS]
    objs = [u[1] for u in units]
    jobs = jobs or min(len(units), max(1, min(os.cpu_count() or 1, 8)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(lambda u: _compile(u[0], u[1], u[2]), units))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + (
        SAN_FLAGS + ["-shared-libsan"] if sanitize else []) + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{res.stdout + res.stderr}")
    os.replace(tmp, lib)
    return lib


def build_probes(verbose: bool = False) -> str:
    """Compile the measurement probes (probes/probes.hip) to libsq_probes.so."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    obj = os.path.join(objdir, "probes.hip.o")
    out = _compile(PROBE_SRC, obj)
    if verbose and out.strip():
        print(out)
    tmp = PROBE_LIB + ".tmp"
    res = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"probe link failed ({res.returncode}):\n{res.stdout + res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    if "--probes" in sys.argv:
        print(build_probes(verbose="-v" in sys.argv))
        sys.exit(0)
    print(build_library(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
