"""Host replay of the int8 GEMM kernels' index arithmetic with bounds checks.

tests/index_replay.cpp compiles the index maps and launch plans the prefill
and decode kernels use (csrc/gemm_index.hpp) with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer, and replays every workgroup's, wave's and
lane's addresses for every template configuration the dispatch launches and
a list of shapes (the workloads' prefill and decode GEMMs and ragged ones):
tile schedule, K slices, direct-to-LDS transfers and fragment reads, split-K
partial tiles and the reducer's reads, epilogue staging and stores. No GPU is
needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "index_replay.cpp")
CSRC = os.path.join(ROOT, "w8a8_int8_quantization_amd", "csrc")


@pytest.mark.timeout(600)
def test_gemm_index_replay(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "index_replay")
    # the sanitizer runtimes are linked statically, so the program runs
    # under whatever the environment preloads
    cmd = [gxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-static-libasan", "-static-libubsan", f"-I{CSRC}", SRC, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=500, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert run.stdout.startswith("OK "), run.stdout
    assert int(run.stdout.split()[1]) > 10**9  # the replay really ran
