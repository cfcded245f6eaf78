"""The C-ABI library loads, exports every entry point declared in include/sq.h,
and rejects bad arguments before touching the GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sq.h")
LIB = os.environ.get("SQ_LIBRARY") or os.path.join(ROOT, "w8a8_int8_quantization_amd", "libsq.so")


@pytest.fixture(scope="module")
def sq():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_sq_build", os.path.join(ROOT, "w8a8_int8_quantization_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build_library()
    import w8a8_int8_quantization_amd as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_core_calls():
    names = declared_functions()
    for core in ("sq_calibrate_absmax", "sq_smooth_fold_weights", "sq_quant_act_per_token", "sq_w8a8_linear"):
        assert core in names


def test_library_exports_every_declared_symbol(sq):
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(sq.EXPORTED_SYMBOLS) == declared_functions()


def test_version_and_status_strings(sq):
    assert sq.sq_version() == 10000
    for st in range(8):
        assert sq.raw["sq_status_string"](st).decode()
    assert sq.raw["sq_status_string"](99).decode() == "unknown status"


OK, NULL, DTYPE, SHAPE, ALIGN, RANGE, WS = 0, 1, 2, 3, 4, 5, 6
P = 1 << 20          # a 16-byte-aligned stand-in address; never dereferenced by these calls
BAD = P + 1


def test_validation_calibrate(sq):
    f = sq.raw["sq_calibrate_absmax"]
    assert f(P, sq.SQ_BF16, 4, 100, 100, P, None) == SHAPE      # K not a multiple of 64
    assert f(P, sq.SQ_BF16, 4, 0, 0, P, None) == SHAPE          # K = 0
    assert f(P, sq.SQ_I8, 4, 64, 64, P, None) == DTYPE
    assert f(None, sq.SQ_F32, 4, 64, 64, P, None) == NULL
    assert f(P, sq.SQ_F32, 4, 64, 64, None, None) == NULL
    assert f(BAD, sq.SQ_F32, 4, 64, 64, P, None) == ALIGN
    assert f(P, sq.SQ_BF16, 4, 64, 68, P, None) == ALIGN        # rows not 16-byte aligned
    assert f(P, sq.SQ_F32, 4, 64, 32, P, None) == SHAPE         # ld < K
    assert f(P, sq.SQ_F32, -1, 64, 64, P, None) == SHAPE
    assert f(None, sq.SQ_F32, 0, 64, 64, P, None) == OK         # empty batch: no work


def test_validation_fold(sq):
    f = sq.raw["sq_smooth_fold_weights"]
    ws = sq.raw["sq_smooth_fold_workspace_size"](128, 100)
    assert ws >= 400 and ws % 256 == 0
    assert f(P, P, sq.SQ_BF16, 128, 100, 104, 1.5, 0, P, P, P, P, ws, None) == RANGE   # alpha > 1
    assert f(P, P, sq.SQ_BF16, 128, 100, 104, -0.1, 0, P, P, P, P, ws, None) == RANGE
    assert f(P, P, sq.SQ_BF16, 128, 100, 104, 0.5, 7, P, P, P, P, ws, None) == RANGE   # flags
    assert f(None, P, sq.SQ_BF16, 128, 100, 104, 0.5, 0, P, P, P, P, ws, None) == NULL  # absmax for COMPUTE
    assert f(P, P, sq.SQ_BF16, 128, 100, 104, 0.5, 1, None, P, P, P, ws, None) == NULL  # smooth for GIVEN
    assert f(P, P, sq.SQ_BF16, 128, 100, 104, 0.5, 0, P, P, P, P, ws - 256, None) == WS
    assert f(P, P + 1, sq.SQ_BF16, 128, 100, 104, 0.5, 0, P, P, P, P, ws, None) == ALIGN  # odd address
    assert f(P, P, sq.SQ_BF16, 128, 100, 99, 0.5, 0, P, P, P, P, ws, None) == SHAPE      # ld < N
    assert f(P, P, sq.SQ_BF16, 100, 100, 104, 0.5, 0, P, P, P, P, ws, None) == SHAPE
    assert f(P, P, sq.SQ_I32, 128, 100, 104, 0.5, 0, P, P, P, P, ws, None) == DTYPE
    assert f(P, P, sq.SQ_BF16, 128, 100, 104, 0.5, 0, P, BAD, P, P, ws, None) == ALIGN


def test_validation_quant(sq):
    f = sq.raw["sq_quant_act_per_token"]
    assert f(P, sq.SQ_BF16, 4, 96, 96, None, P, P, None) == SHAPE
    assert f(P, sq.SQ_BF16, 4, 64, 64, None, None, P, None) == NULL
    assert f(P, sq.SQ_BF16, 4, 64, 64, None, P, None, None) == NULL
    assert f(P, sq.SQ_BF16, 4, 64, 64, BAD, P, P, None) == ALIGN
    assert f(P, sq.SQ_BF16, 4, 64, 64, None, BAD, P, None) == ALIGN
    assert f(None, sq.SQ_BF16, 0, 64, 64, None, None, None, None) == OK
    g = sq.raw["sq_quant_act_rows_masked"]
    assert g(P, sq.SQ_F16, 4, 64, 64, None, P, P, None) == NULL


def test_validation_linear(sq):
    f = sq.raw["sq_w8a8_linear"]
    assert sq.raw["sq_w8a8_linear_workspace_size"](2048, 6144, 4096) == 0
    kmax = sq.MAX_K_INT32
    assert 127 * 127 * kmax < 2 ** 31 <= 127 * 127 * (kmax + 1)
    big_k = (kmax // 64 + 1) * 64
    assert f(P, P, P, P, 4, 4, big_k, P, sq.SQ_BF16, 4, None, 0, None) == RANGE
    assert f(P, P, P, P, 4, 4, 100, P, sq.SQ_BF16, 4, None, 0, None) == SHAPE
    assert f(P, P, P, P, 4, 4, 64, P, sq.SQ_I8, 4, None, 0, None) == DTYPE
    assert f(P, P, P, P, 4, 8, 64, P, sq.SQ_BF16, 4, None, 0, None) == SHAPE   # ldy < N
    assert f(None, P, P, P, 4, 4, 64, P, sq.SQ_BF16, 4, None, 0, None) == NULL
    assert f(P, None, P, P, 4, 4, 64, P, sq.SQ_BF16, 4, None, 0, None) == NULL
    assert f(BAD, P, P, P, 4, 4, 64, P, sq.SQ_BF16, 4, None, 0, None) == ALIGN
    assert f(P, P, P, P, 4, 4, 64, BAD, sq.SQ_BF16, 4, None, 0, None) == ALIGN   # odd address for bf16
    assert f(None, None, None, None, 0, 4, 64, None, sq.SQ_BF16, 4, None, 0, None) == OK
    # decode shapes split K: workspace required, 16-byte aligned
    need = sq.raw["sq_w8a8_linear_workspace_size"](4, 4096, 14336)
    assert need >= 4 * 4 * 4096 * 2
    assert f(P, P, P, P, 4, 4096, 14336, P, sq.SQ_BF16, 4096, None, 0, None) == WS
    assert f(P, P, P, P, 4, 4096, 14336, P, sq.SQ_BF16, 4096, P, need - 1, None) == WS
    assert f(P, P, P, P, 4, 4096, 14336, P, sq.SQ_BF16, 4096, BAD, need, None) == ALIGN
    # 65..256 tokens: the decode kernel only where the tiled kernels get few tiles
    assert sq.raw["sq_w8a8_linear_workspace_size"](128, 4096, 14336) > 0       # down projection shape
    # 160..255 tokens over wide layers: the 256-row kernel, K split 3 ways over
    # its 75 tiles of 256 x 192, the partial tiles after the fixed 1 KiB
    # counter region
    assert sq.raw["sq_w8a8_linear_workspace_size"](192, 14336, 4096) == 1024 + 3 * 75 * 256 * 192 * 4
    assert sq.raw["sq_w8a8_linear_workspace_size"](150, 20000, 2048) == 0      # 128 x 128 tiles
    # prefill with 2 x 22 tiles of 256 x 192: K (112 stages of 128) split 5
    # ways, 5 x 44 partial int32 tiles after the counter region
    assert sq.raw["sq_w8a8_linear_workspace_size"](257, 4096, 14336) == 1024 + 5 * 44 * 256 * 192 * 4
    # decode: 64 columns x 64 tokens per counter, partial tiles [S][M][N] after the region
    assert sq.raw["sq_w8a8_linear_workspace_size"](64, 4096, 14336) == 1024 + 4 * 64 * 4096 * 4
    assert sq.raw["sq_w8a8_linear_workspace_size"](4096, 4096, 14336) == 0     # 256 tiles: no split
    d = sq.raw["sq_w8a8_linear_dyn"]
    need = sq.raw["sq_w8a8_linear_dyn_workspace_size"](4, 4, 64)
    assert need >= 4 * 64 + 16
    assert d(P, sq.SQ_BF16, 64, None, P, P, 4, 4, 64, P, sq.SQ_BF16, 4, P, need - 1, None) == WS
    assert d(P, sq.SQ_BF16, 64, None, P, P, 4, 4, 64, P, sq.SQ_I32, 4, P, need, None) == DTYPE


def test_validation_llm_int8(sq):
    f = sq.raw["sq_int8_decomp_linear"]
    need = sq.raw["sq_int8_decomp_workspace_size"](4096, 8192, 8192)
    assert need >= 4096 * 8192 + 4096 * 4 + 8192 * 9
    args = [P, 64, P, P, P, 64, 4, 64, 64, 6.0, P, 64, P, P, need, None]
    assert f(*args[:9], float("nan"), *args[10:]) == RANGE
    a = list(args); a[12] = None
    assert f(*a) == NULL
    a = list(args); a[14] = 16
    assert f(*a) == WS
    g = sq.raw["sq_outlier_detect"]
    assert g(P, sq.SQ_F16, 4, 64, 64, 6.0, None, P, P, P, 256, None) == NULL
    assert g(P, sq.SQ_F16, 4, 64, 64, 6.0, P, P, P, P, 0, None) == WS


def test_validation_decomp_gemm(sq):
    f = sq.raw["sq_int8_decomp_gemm"]
    args = [P, P, P, 64, P, P, P, 64, P, P, 4, 64, 64, P, 64, None]
    a = list(args); a[0] = None
    assert f(*a) == NULL
    a = list(args); a[8] = None
    assert f(*a) == NULL
    a = list(args); a[3] = 32   # ldx < k
    assert f(*a) == SHAPE
    a = list(args); a[12] = 100  # k not a multiple of 64
    assert f(*a) == SHAPE
    a = list(args); a[0] = BAD
    assert f(*a) == ALIGN
    a = list(args); a[13] = P + 1  # odd fp16 output address
    assert f(*a) == ALIGN
    a = list(args); a[10] = 0
    assert f(*a) == OK


def test_validation_rmsnorm(sq):
    f = sq.raw["sq_rmsnorm_quant"]
    assert f(P, sq.SQ_BF16, 4, 100, 100, P, 1e-5, P, P, None) == SHAPE        # K not a multiple of 64
    assert f(P, sq.SQ_BF16, 4, 32768 + 64, 32768 + 64, P, 1e-5, P, P, None) == RANGE  # beyond SQ_MAX_K_NORM
    assert f(P, sq.SQ_I8, 4, 64, 64, P, 1e-5, P, P, None) == DTYPE
    assert f(P, sq.SQ_BF16, 4, 64, 64, P, -1.0, P, P, None) == RANGE         # eps < 0
    assert f(P, sq.SQ_BF16, 4, 64, 64, P, float("inf"), P, P, None) == RANGE
    assert f(P, sq.SQ_BF16, 4, 64, 64, P, float("nan"), P, P, None) == RANGE
    assert f(P, sq.SQ_BF16, 4, 64, 64, None, 0.0, P, P, None) == NULL        # gain
    assert f(P, sq.SQ_BF16, 4, 64, 64, P, 0.0, None, P, None) == NULL
    assert f(P, sq.SQ_BF16, 4, 64, 64, P, 0.0, P, None, None) == NULL
    assert f(P, sq.SQ_BF16, 4, 64, 64, BAD, 0.0, P, P, None) == ALIGN        # gain alignment
    assert f(P, sq.SQ_BF16, 4, 64, 64, P, 0.0, BAD, P, None) == ALIGN
    assert f(P, sq.SQ_BF16, 4, 64, 68, P, 0.0, P, P, None) == ALIGN          # row pitch
    assert f(None, sq.SQ_BF16, 0, 64, 64, None, 0.0, None, None, None) == OK  # empty batch: no work
    g = sq.raw["sq_fold_norm_gain"]
    assert g(P, sq.SQ_I8, P, 64, P, None) == DTYPE
    assert g(None, sq.SQ_BF16, P, 64, P, None) == NULL
    assert g(P, sq.SQ_BF16, P, 64, None, None) == NULL
    assert g(P + 1, sq.SQ_BF16, P, 64, P, None) == ALIGN
    assert g(P, sq.SQ_F32, P + 2, 64, P, None) == ALIGN
    assert g(P, sq.SQ_BF16, P, -1, P, None) == SHAPE
    assert g(None, sq.SQ_BF16, None, 0, None, None) == OK
    h = sq.raw["sq_rmsnorm_w8a8_linear"]
    nb = sq.raw["sq_rmsnorm_w8a8_linear_workspace_size"](16, 128, 256)
    assert nb == sq.raw["sq_w8a8_linear_dyn_workspace_size"](16, 128, 256) > 0
    assert h(P, sq.SQ_BF16, 256, P, 0.0, P, P, 16, 128, 256, P, sq.SQ_I32, 128, P, nb, None) == DTYPE
    assert h(P, sq.SQ_BF16, 256, P, 0.0, P, P, 16, 128, 256, P, sq.SQ_BF16, 128, P, nb - 1, None) == WS
    assert h(P, sq.SQ_BF16, 256, P, 0.0, P, P, 16, 128, 256, P, sq.SQ_BF16, 128, None, 0, None) == WS
    assert h(P, sq.SQ_BF16, 256, P, -2.0, P, P, 16, 128, 256, P, sq.SQ_BF16, 128, P, nb, None) == RANGE
    assert h(P, sq.SQ_BF16, 256, None, 0.0, P, P, 16, 128, 256, P, sq.SQ_BF16, 128, P, nb, None) == NULL
    assert h(P, sq.SQ_BF16, 256, P, 0.0, None, P, 16, 128, 256, P, sq.SQ_BF16, 128, P, nb, None) == NULL
    assert h(P, sq.SQ_BF16, 256, P, 0.0, P, P, 16, 128, 256, P, sq.SQ_BF16, 100, P, nb, None) == SHAPE


def test_validation_silu(sq):
    f = sq.raw["sq_silu_mul_quant"]
    assert f(P, P, sq.SQ_BF16, 4, 100, 100, 100, None, P, P, None) == SHAPE       # K not a multiple of 64
    assert f(P, P, sq.SQ_BF16, 4, 32768 + 64, 32768 + 64, 32768 + 64, None, P, P, None) == RANGE
    assert f(P, P, sq.SQ_F16, 4, 64, 64, 64, None, P, P, None) == DTYPE           # bf16 only
    assert f(P, P, sq.SQ_F32, 4, 64, 64, 64, None, P, P, None) == DTYPE
    assert f(None, P, sq.SQ_BF16, 4, 64, 64, 64, None, P, P, None) == NULL
    assert f(P, None, sq.SQ_BF16, 4, 64, 64, 64, None, P, P, None) == NULL
    assert f(P, P, sq.SQ_BF16, 4, 64, 64, 64, None, None, P, None) == NULL
    assert f(P, P, sq.SQ_BF16, 4, 64, 64, 64, None, P, None, None) == NULL
    assert f(BAD, P, sq.SQ_BF16, 4, 64, 64, 64, None, P, P, None) == ALIGN
    assert f(P, P, sq.SQ_BF16, 4, 64, 64, 68, None, P, P, None) == ALIGN         # up rows not 16-byte aligned
    assert f(P, P, sq.SQ_BF16, 4, 64, 64, 64, BAD, P, P, None) == ALIGN          # smooth
    assert f(P, P, sq.SQ_BF16, 4, 64, 64, 32, None, P, P, None) == SHAPE         # ld < K
    assert f(None, None, sq.SQ_BF16, 0, 64, 64, 64, None, None, None, None) == OK  # empty batch
    h = sq.raw["sq_silu_mul_w8a8_linear"]
    nb = sq.raw["sq_silu_mul_w8a8_linear_workspace_size"](16, 128, 256)
    assert nb == sq.raw["sq_w8a8_linear_dyn_workspace_size"](16, 128, 256) > 0
    assert h(P, P, sq.SQ_BF16, 256, 256, None, P, P, 16, 128, 256, P, sq.SQ_I32, 128, P, nb, None) == DTYPE
    assert h(P, P, sq.SQ_BF16, 256, 256, None, P, P, 16, 128, 256, P, sq.SQ_BF16, 128, P, nb - 1, None) == WS
    assert h(P, P, sq.SQ_F16, 256, 256, None, P, P, 16, 128, 256, P, sq.SQ_BF16, 128, P, nb, None) == DTYPE
    assert h(P, P, sq.SQ_BF16, 256, 256, None, None, P, 16, 128, 256, P, sq.SQ_BF16, 128, P, nb, None) == NULL


def test_validation_fp8(sq):
    f = sq.raw["sq_quant_act_fp8"]
    assert f(P, sq.SQ_BF16, 4, 100, 100, P, P, None) == SHAPE
    assert f(P, sq.SQ_BF16, 4, 32768 + 64, 32768 + 64, P, P, None) == RANGE
    assert f(P, sq.SQ_I8, 4, 64, 64, P, P, None) == DTYPE
    assert f(P, sq.SQ_BF16, 4, 64, 64, None, P, None) == NULL
    assert f(P, sq.SQ_BF16, 4, 64, 64, BAD, P, None) == ALIGN
    assert f(None, sq.SQ_BF16, 0, 64, 64, None, None, None) == OK
    g = sq.raw["sq_quant_weights_fp8"]
    nb = sq.raw["sq_quant_weights_fp8_workspace_size"](128, 192)
    assert nb >= 192 * 4
    assert g(P, sq.SQ_BF16, 128, 100, 100, P, P, P, nb, None) == SHAPE      # N % 64
    assert g(P, sq.SQ_BF16, 128, 192, 192, P, P, P, nb - 1, None) == WS
    assert g(P, sq.SQ_BF16, 128, 192, 192, None, P, P, nb, None) == NULL
    assert g(P, sq.SQ_BF16, 128, 192, 196, P, P, P, nb, None) == ALIGN      # row pitch
    h = sq.raw["sq_fp8_linear"]
    nbw = sq.raw["sq_fp8_linear_workspace_size"](4, 64, 256)
    assert nbw > 0                                                          # decode shape, K split
    assert nbw == sq.raw["sq_w8a8_linear_workspace_size"](4, 64, 256)
    assert sq.raw["sq_fp8_linear_workspace_size"](2048, 6144, 4096) == 0
    assert h(P, P, P, P, 4, 64, 192, P, sq.SQ_BF16, 64, P, nbw, None) == SHAPE      # K % 128
    assert h(P, P, P, P, 4, 64, 32768 + 128, P, sq.SQ_BF16, 64, P, nbw, None) == RANGE
    assert h(P, P, P, P, 4, 64, 256, P, sq.SQ_I32, 64, P, nbw, None) == DTYPE
    assert h(None, P, P, P, 4, 64, 256, P, sq.SQ_BF16, 64, P, nbw, None) == NULL
    assert h(P, P, P, P, 4, 64, 256, P, sq.SQ_BF16, 32, P, nbw, None) == SHAPE      # ldy < N
    assert h(P, P, P, P, 4, 64, 256, P, sq.SQ_BF16, 64, P, nbw - 1, None) == WS
    assert h(P, P, P, P, 4, 64, 256, P, sq.SQ_BF16, 64, None, 0, None) == WS
    assert h(P, P, P, P, 4, 64, 256, P, sq.SQ_BF16, 64, BAD, nbw, None) == ALIGN
    assert h(None, None, None, None, 0, 64, 256, None, sq.SQ_BF16, 64, None, 0, None) == OK
    dyn = sq.raw["sq_fp8_linear_dyn"]
    nbd = sq.raw["sq_fp8_linear_dyn_workspace_size"](4, 64, 256)
    assert dyn(P, sq.SQ_BF16, 256, P, P, 4, 64, 256, P, sq.SQ_BF16, 64, P, nbd - 1, None) == WS


def test_validation_gptq(sq):
    f = sq.raw["sq_gptq_hessian"]
    assert f(P, sq.SQ_BF16, 16, 192, 192, None, P, None) == SHAPE            # K % 128
    assert f(P, sq.SQ_BF16, 16, 32768 + 128, 32768 + 128, None, P, None) == RANGE
    assert f(P, sq.SQ_I8, 16, 128, 128, None, P, None) == DTYPE
    assert f(P, sq.SQ_BF16, 16, 128, 100, None, P, None) == SHAPE            # ldx < K
    assert f(P, sq.SQ_BF16, 16, 128, 128, None, None, None) == NULL
    assert f(P, sq.SQ_BF16, 16, 128, 128, None, P + 4, None) == ALIGN        # h not 8-byte aligned
    assert f(None, sq.SQ_BF16, 0, 128, 128, None, None, None) == OK          # no rows: nothing to do
    g = sq.raw["sq_gptq_quantize"]
    nb = sq.raw["sq_gptq_quantize_workspace_size"](256, 96)
    assert nb >= 256 * 256 * 8 + 12 * 256 * 96
    assert sq.raw["sq_gptq_quantize_workspace_size"](0, 96) == 0
    assert g(P, P, sq.SQ_BF16, 192, 96, 96, None, 0.01, P, P, P, nb, None) == SHAPE      # K % 128
    assert g(P, P, sq.SQ_BF16, 256, 96, 64, None, 0.01, P, P, P, nb, None) == SHAPE      # ldw < N
    assert g(P, P, sq.SQ_BF16, 256, 96, 96, None, 0.0, P, P, P, nb, None) == RANGE       # damp
    assert g(P, P, sq.SQ_BF16, 256, 96, 96, None, 1.5, P, P, P, nb, None) == RANGE
    assert g(P, P, sq.SQ_I32, 256, 96, 96, None, 0.01, P, P, P, nb, None) == DTYPE
    assert g(None, P, sq.SQ_BF16, 256, 96, 96, None, 0.01, P, P, P, nb, None) == NULL
    assert g(P, P, sq.SQ_BF16, 256, 96, 96, None, 0.01, BAD, P, P, nb, None) == ALIGN    # wq 16-byte
    assert g(P, P, sq.SQ_BF16, 256, 96, 96, None, 0.01, P, P, P, nb - 1, None) == WS
    assert g(P, P, sq.SQ_BF16, 256, 96, 96, None, 0.01, P, P, BAD, nb, None) == ALIGN
    assert g(None, None, sq.SQ_BF16, 256, 0, 0, None, 0.01, None, None, None, 0, None) == OK


def test_out_of_range_enums_rejected(sq):
    """A C caller may pass any int for an enum argument: out-of-range element
    types are rejected with SQ_ERR_DTYPE before anything else is looked at, and
    an unknown status has a string (the host-sanitized build checks that no
    such value is ever loaded as the enum)."""
    r, BADT = sq.raw, 17
    assert r["sq_status_string"](-5).decode() == "unknown status"
    calls = [
        ("sq_calibrate_absmax", (P, BADT, 4, 64, 64, P, None)),
        ("sq_smooth_fold_weights", (P, P, BADT, 64, 64, 64, 0.5, 0, P, P, P, P, 1 << 20, None)),
        ("sq_quant_act_per_token", (P, BADT, 4, 64, 64, None, P, P, None)),
        ("sq_w8a8_linear", (P, P, P, P, 4, 64, 64, P, BADT, 64, None, 0, None)),
        ("sq_w8a8_linear_dyn", (P, BADT, 64, None, P, P, 4, 64, 64, P, sq.SQ_BF16, 64, P, 1 << 20, None)),
        ("sq_w8a8_linear_dyn", (P, sq.SQ_BF16, 64, None, P, P, 4, 64, 64, P, BADT, 64, P, 1 << 20, None)),
        ("sq_w8a8_linear_dyn_static", (P, BADT, 64, None, P, P, 4, 64, 64, P, sq.SQ_BF16, 64, None)),
        ("sq_fold_norm_gain", (P, BADT, None, 64, P, None)),
        ("sq_rmsnorm_quant", (P, BADT, 4, 64, 64, P, 1e-5, P, P, None)),
        ("sq_silu_mul_quant", (P, P, BADT, 4, 64, 64, 64, None, P, P, None)),
        ("sq_quant_act_fp8", (P, BADT, 4, 64, 64, P, P, None)),
        ("sq_fp8_linear", (P, P, P, P, 4, 64, 128, P, BADT, 64, None, 0, None)),
        ("sq_gptq_hessian", (P, BADT, 4, 128, 128, None, P, None)),
        ("sq_outlier_detect", (P, BADT, 4, 64, 64, 6.0, P, P, P, P, 1 << 20, None)),
        ("sq_quant_act_rows_masked", (P, BADT, 4, 64, 64, P, P, P, None)),
    ]
    for name, args in calls:
        assert r[name](*args) == DTYPE, name
