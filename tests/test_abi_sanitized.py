"""The C-ABI tests again, against the host-sanitized build of the library
(AddressSanitizer + UndefinedBehaviorSanitizer on the host code, gfx950 device
code as usual): every argument check, size computation and error path of the
entry points runs with out-of-bounds, overflow and invalid-enum-load detection
on. No compute call is made, so no GPU is needed."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "w8a8_int8_quantization_amd")


def _build_module():
    spec = importlib.util.spec_from_file_location("_sq_build_san", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _stale(lib: str, b) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    import glob
    srcs = list(b.sources()) + glob.glob(os.path.join(PKG, "csrc", "*.hpp")) + [
        os.path.join(ROOT, "include", "sq.h")]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.mark.timeout(900)
def test_abi_checks_clean_under_asan_ubsan():
    b = _build_module()
    if _stale(b.SAN_LIB, b):
        b.build_library(sanitize=True)
    rt = b.asan_runtime()
    if not rt or not os.path.exists(rt):
        pytest.skip("clang AddressSanitizer runtime not found")
    env = dict(os.environ)
    # the AddressSanitizer runtime must come first; whatever the environment
    # already preloads stays after it
    pre = os.environ.get("LD_PRELOAD", "")
    env.update(
        LD_PRELOAD=rt + (":" + pre if pre else ""),
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
        UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
        SQ_LIBRARY=b.SAN_LIB,
    )
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi_cpu.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "runtime error" not in out, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
