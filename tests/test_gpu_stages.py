"""Stage-by-stage parity of the HIP path with the CPU oracle on small and ragged shapes.

Integer and byte results (absmax, Wq, Xq, scales, int32 accumulators, masks,
counts) must be bit-exact; smoothing factors within 1 binary32 ulp; outputs
within 1 ulp of the output type. Every call goes through the C ABI via the
ctypes binding.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import (assert_out_close, bits16, dev, host, log, padded, to_dev, ulp_diff32)

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("w8a8_int8_quantization_amd")


# --------------------------------------------------------------------------- calibration
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("t,k", [(1, 64), (7, 192), (64, 256), (1000, 4160), (37, 14336)])
def test_calibrate_absmax(dtype, t, k):
    log("calibrate", dtype, t, k)
    c = workloads.random_linear_case(m=1, k=k, n=64, seed=t + k, dtype=dtype if dtype != "f16" else "f16",
                                     calib_rows=t)
    xc = to_dev(c.x_calib, dtype)
    a = torch.zeros(k, dtype=torch.float32, device=dev())
    sq.sq_calibrate_absmax(xc, a)
    assert np.array_equal(host(a), oracle.calibrate_absmax(c.x_calib))
    # running maximum across two batches, with a padded leading dimension
    half = t // 2
    a2 = torch.zeros(k, dtype=torch.float32, device=dev())
    if half:
        sq.sq_calibrate_absmax(padded(c.x_calib[:half], dtype, k + 64), a2)
    sq.sq_calibrate_absmax(to_dev(c.x_calib[half:], dtype), a2)
    assert np.array_equal(host(a2), oracle.calibrate_absmax(c.x_calib[half:], oracle.calibrate_absmax(c.x_calib[:half])))


# --------------------------------------------------------------------------- weight fold
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("k,n,alpha", [(64, 1, 0.5), (128, 100, 0.5), (256, 512, 0.8), (448, 1000, 0.0),
                                       (320, 72, 1.0), (4096, 520, 0.5), (192, 333, 0.5)])
@pytest.mark.parametrize("aligned_rows", [True, False])
def test_smooth_fold(dtype, k, n, alpha, aligned_rows):
    log("fold", dtype, k, n, alpha, aligned_rows)
    c = workloads.random_linear_case(m=4, k=k, n=n, seed=k * 7 + n, dtype=dtype, calib_rows=96, alpha=alpha)
    a_ref = oracle.calibrate_absmax(c.x_calib)
    # padded 16-byte aligned rows, or rows of exactly N elements (any pitch)
    ld = (n + 7) // 8 * 8 + 8 if aligned_rows else n
    w = padded(c.w, dtype, ld)
    a = torch.from_numpy(a_ref).to(dev())
    s, wq, sw = sq.sq_smooth_fold_weights(w, alpha, absmax=a)
    s_ref = oracle.smoothing_factors(a_ref, oracle.weight_row_absmax(c.w), alpha)
    d = ulp_diff32(host(s), s_ref)
    assert d.max() <= 1, f"s differs by {d.max()} ulp"
    log("  s exact fraction", float((d == 0).mean()))
    # with the oracle's s given to both sides every later value is bit-exact
    s_in = torch.from_numpy(s_ref).to(dev())
    _, wq, sw = sq.sq_smooth_fold_weights(w, smooth=s_in, flags=sq.SMOOTH_GIVEN)
    wq_ref, sw_ref = oracle.quantize_weights_per_channel(oracle.fold_weights(c.w, s_ref))
    assert np.array_equal(host(wq), wq_ref)
    assert np.array_equal(host(sw), sw_ref)
    # no smoothing: plain per-channel weight quantisation
    _, wq0, sw0 = sq.sq_smooth_fold_weights(w, flags=sq.SMOOTH_NONE)
    wq0_ref, sw0_ref = oracle.quantize_weights_per_channel(c.w)
    assert np.array_equal(host(wq0), wq0_ref) and np.array_equal(host(sw0), sw0_ref)


def test_smooth_fold_zero_rows_and_columns():
    k, n = 128, 96
    c = workloads.random_linear_case(m=4, k=k, n=n, seed=5, dtype="f32", calib_rows=32)
    w = c.w.copy()
    w[5] = 0          # W_j = 0 -> s_j = 1
    w[:, 7] = 0       # zero column -> sw = 0, Wq column = 0
    a_ref = oracle.calibrate_absmax(c.x_calib)
    a_ref[9] = 0      # A_j = 0 -> s_j = 1
    s, wq, sw = sq.sq_smooth_fold_weights(to_dev(w, "f32"), 0.5, absmax=torch.from_numpy(a_ref).to(dev()))
    s_ref, wq_ref, sw_ref = oracle.smooth_fold_quantize(a_ref, w, 0.5)
    assert host(s)[5] == 1 and host(s)[9] == 1
    assert ulp_diff32(host(s), s_ref).max() <= 1
    _, wq, sw = sq.sq_smooth_fold_weights(to_dev(w, "f32"), smooth=torch.from_numpy(s_ref).to(dev()),
                                          flags=sq.SMOOTH_GIVEN)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(sw), sw_ref)
    assert host(sw)[7] == 0 and np.all(host(wq)[7] == 0)


# --------------------------------------------------------------------------- activation quant
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("m,k", [(1, 64), (3, 256), (257, 512), (33, 4096), (5, 14336), (9, 16384), (4, 20480)])
@pytest.mark.parametrize("smooth", [False, True])
def test_quant_act(dtype, m, k, smooth):
    log("quant", dtype, m, k, smooth)
    c = workloads.random_linear_case(m=m, k=k, n=64, seed=m * 31 + k, dtype=dtype, calib_rows=64)
    x = c.x.copy()
    if m > 2:
        x[1] = 0  # zero row -> scale 0, Xq row 0
    s_ref = None
    if smooth:
        s_ref = oracle.smoothing_factors(oracle.calibrate_absmax(c.x_calib), oracle.weight_row_absmax(c.w), 0.5)
    xq, dx = sq.sq_quant_act_per_token(to_dev(x, dtype), None if s_ref is None else torch.from_numpy(s_ref).to(dev()))
    xq_ref, dx_ref = oracle.quantize_activations(x, s_ref)
    assert np.array_equal(host(dx), dx_ref)
    assert np.array_equal(host(xq), xq_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("k", [64, 192, 4096, 4160, 8192, 14336, 16384])
@pytest.mark.parametrize("smooth", [False, True])
def test_quant_act_prefill_kernel(dtype, k, smooth):
    """A few hundred rows of every row length the kernels distinguish."""
    if dtype == "f32" and k > 8192:
        pytest.skip("covered by the workgroup-per-row kernel")
    m = 133
    log("quant wave", dtype, k, smooth)
    c = workloads.random_linear_case(m=m, k=k, n=64, seed=k + m + int(smooth), dtype=dtype, calib_rows=64,
                                     model="silu_gated" if k > 8192 else "gaussian_outlier")
    x = c.x.copy()
    x[3] = 0
    s_ref = None
    if smooth:
        s_ref = oracle.smoothing_factors(oracle.calibrate_absmax(c.x_calib), oracle.weight_row_absmax(c.w), 0.5)
    xq, dx = sq.sq_quant_act_per_token(to_dev(x, dtype), None if s_ref is None else torch.from_numpy(s_ref).to(dev()))
    xq_ref, dx_ref = oracle.quantize_activations(x, s_ref)
    assert np.array_equal(host(dx), dx_ref)
    assert np.array_equal(host(xq), xq_ref)


@pytest.mark.parametrize("m,k", [(3, 16384), (1, 4096), (64, 8192), (1100, 4096), (1030, 16384), (1100, 14336)])
@pytest.mark.parametrize("hi_exp", [20, 21])
def test_quant_act_smooth_spread(m, k, hi_exp):
    """Smoothing factors with random significands over every binade of the
    fast-division range (2^-20 .. 2^20, edge significands included): the
    per-column reciprocals and quotients must reproduce IEEE division exactly.
    hi_exp 21 puts some factors past the fast range (IEEE fallback)."""
    log("quant spread", m, k, hi_exp)
    ch = workloads.outlier_channels(k, seed=k)
    x = workloads.activations(m, k, "gaussian_outlier", seed=m + k, role="x", channels=ch, dtype="bf16")
    s = workloads.spread_scales(k, seed=m + k + hi_exp, hi_exp=hi_exp)
    xq, dx = sq.sq_quant_act_per_token(to_dev(x, "bf16"), torch.from_numpy(s).to(dev()))
    xq_ref, dx_ref = oracle.quantize_activations(x, s)
    assert np.array_equal(host(dx), dx_ref)
    assert np.array_equal(host(xq), xq_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_act_range_fallbacks(dtype):
    """Rows and smoothing factors outside the fast-division bounds take IEEE division
    and still match the oracle bit for bit: tiny rows, huge rows, rows mixing tiny
    and normal values, and smoothing factors far from 1."""
    m, k = 96, 512
    rng = np.random.default_rng(77)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[0] *= np.float32(1e-35)                     # whole row tiny: d < 2^-30
    x[1] *= np.float32(1e25)                      # huge row: max > 2^50
    x[2, ::3] *= np.float32(1e-30)                # tiny entries inside a normal row
    x[3, 5] = np.float32(3e-39)                   # a subnormal entry
    x[4] = 0
    x[5, :7] = [1e-20, -2e-25, 5e-30, 1e-38, 2e-40, -7e-42, 0]
    xr = oracle.round_bf16(x) if dtype == "bf16" else x
    for s_ref in (None, np.exp(rng.uniform(-2, 2, k)).astype(np.float32)):
        xq, dx = sq.sq_quant_act_per_token(to_dev(xr, dtype), None if s_ref is None else torch.from_numpy(s_ref).to(dev()))
        xq_ref, dx_ref = oracle.quantize_activations(xr, s_ref)
        assert np.array_equal(host(dx), dx_ref) and np.array_equal(host(xq), xq_ref)
    # smoothing factors outside [2^-20, 2^20] switch the whole launch to IEEE division
    s_bad = np.exp(rng.uniform(-2, 2, k)).astype(np.float32)
    s_bad[17] = np.float32(1e-8)
    s_bad[18] = np.float32(3e7)
    xq, dx = sq.sq_quant_act_per_token(to_dev(xr, dtype), torch.from_numpy(s_bad).to(dev()))
    xq_ref, dx_ref = oracle.quantize_activations(xr, s_bad)
    assert np.array_equal(host(dx), dx_ref) and np.array_equal(host(xq), xq_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("nvec", [256, 512, 1024, 1792])
@pytest.mark.parametrize("m", [1030, 2050])
@pytest.mark.parametrize("smooth", [False, True])
def test_quant_act_full_rows(dtype, nvec, m, smooth):
    """Prefill rows of exactly 1, 2 or 4 16-byte vectors per thread of 256, or
    4 per thread of 448 (the full-row kernel, a workgroup visiting one to five
    rows): zero rows, rows
    outside the fast-division range (all tiny; huge), tiny entries inside
    normal rows, exact .5 quotients, every row checked bit for bit."""
    k = nvec * (4 if dtype == "f32" else 8)
    log("quant full rows", dtype, m, k, smooth)
    rng = np.random.default_rng(m + k + int(smooth))
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, ::97] *= np.float32(20.0)                          # outlier columns
    x[1] = 0
    x[2] *= np.float32(1e-7 if dtype == "f16" else 1e-35)   # whole row tiny: d < 2^-30
    if dtype != "f16":
        x[3] *= np.float32(1e25)                            # max > 2^50
    x[4, ::3] *= np.float32(1e-30 if dtype != "f16" else 1e-6)
    x[5, :] = 0
    x[5, 0] = 127.0
    x[5, 1:9] = [0.5, 1.5, 2.5, -0.5, -2.5, 125.5, -126.5, 64.5]
    x[m - 1] = 0
    xr = oracle.round_bf16(x) if dtype == "bf16" else (x.astype(np.float16).astype(np.float32) if dtype == "f16" else x)
    s_ref = np.exp(rng.uniform(-3, 3, k)).astype(np.float32) if smooth else None
    if smooth:
        s_ref[5] = np.float32(1.0)
    xq, dx = sq.sq_quant_act_per_token(to_dev(xr, dtype), None if s_ref is None else torch.from_numpy(s_ref).to(dev()))
    xq_ref, dx_ref = oracle.quantize_activations(xr, s_ref)
    assert np.array_equal(host(dx), dx_ref)
    assert np.array_equal(host(xq), xq_ref)


@pytest.mark.parametrize("k,nout", [(512, 3), (4096, 8), (8192, 0)])
def test_quant_rows_masked_prefill_kernel(k, nout):
    cfg = workloads.decomp_case(seed=k + nout, m=200, k=k, n=64, n_outlier_cols=nout)
    xh = to_dev(cfg.x, "f16")
    mask_ref = oracle.detect_outliers(cfg.x, 6.0)
    xq, dx = sq.sq_quant_act_rows_masked(xh, torch.from_numpy(mask_ref.astype(np.uint8)).to(dev()))
    xq_ref, dx_ref = oracle.quantize_rows_regular(cfg.x, mask_ref)
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(dx), dx_ref)


def test_quant_act_ties_and_padding():
    """Exact .5 quotients round to even; a padded leading dimension is honoured."""
    k = 128
    row = np.zeros(k, np.float32)
    row[0] = 127.0
    row[1:11] = [0.5, 1.5, 2.5, -0.5, -2.5, 3.5, 125.5, -126.5, 64.5, 0.25]
    x = np.stack([row, -row, row * 2.0 ** -20, row * 2.0 ** 20])
    for dtype in ("f32", "bf16"):
        xq, dx = sq.sq_quant_act_per_token(padded(x, dtype, k + 64))
        xq_ref, dx_ref = oracle.quantize_activations(oracle.round_bf16(x) if dtype == "bf16" else x)
        assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(dx), dx_ref)


# --------------------------------------------------------------------------- int8 GEMM
# Small shapes run the 128 x 128 kernel; from about a million outputs on, the
# 256-row kernel (BN 256, 192 or 128), including ragged M and N tails.
GEMM_SHAPES = [(1, 1, 64), (3, 5, 64), (16, 512, 256), (100, 72, 192), (129, 257, 320), (256, 256, 512),
               (300, 130, 4096), (77, 1000, 1088), (1, 4096, 14336), (64, 200, 14336),
               (1000, 1100, 384), (513, 2050, 1024), (2048, 768, 256), (256, 4096, 128), (777, 1536, 4160),
               (1000, 6100, 1024), (2048, 4096, 4096), (3072, 4096, 512)]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_int32_exact(m, n, k):
    log("gemm i32", m, n, k)
    xq = workloads.uniform_int8((m, k), seed=m + n + k, stream=0)
    wq = workloads.uniform_int8((n, k), seed=m + n + k, stream=1)
    acc = sq.sq_w8a8_linear(torch.from_numpy(xq).to(dev()), None, torch.from_numpy(wq).to(dev()), None,
                            out_dtype=torch.int32)
    assert np.array_equal(host(acc), oracle.int8_matmul(xq, wq))


def test_gemm_extremes():
    """All +-127 at the largest configuration K: |acc| = 231,225,344 exactly."""
    k = 14336
    xq = np.full((70, k), 127, np.int8)
    xq[1::2] = -127
    wq = np.full((130, k), 127, np.int8)
    wq[::3, ::2] = -127
    acc = sq.sq_w8a8_linear(torch.from_numpy(xq).to(dev()), None, torch.from_numpy(wq).to(dev()), None,
                            out_dtype=torch.int32)
    ref = oracle.int8_matmul(xq, wq)
    assert np.abs(ref).max() == 231225344
    assert np.array_equal(host(acc), ref)


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(5, 64, 128), (129, 257, 320), (200, 300, 4096), (1000, 1100, 384),
                                   (512, 2048, 256), (1000, 6100, 1024)])
def test_gemm_dequant(out, m, n, k):
    log("gemm dequant", out, m, n, k)
    xq = workloads.uniform_int8((m, k), seed=3 * m + n, stream=2)
    wq = workloads.uniform_int8((n, k), seed=3 * m + n, stream=3)
    dx = workloads.positive_scales(m, seed=m, stream=0)
    dw = workloads.positive_scales(n, seed=n, stream=1) * np.float32(1e-3)
    y = sq.sq_w8a8_linear(torch.from_numpy(xq).to(dev()), torch.from_numpy(dx).to(dev()),
                          torch.from_numpy(wq).to(dev()), torch.from_numpy(dw).to(dev()),
                          out_dtype={"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out])
    ref = oracle.w8a8_linear(xq, dx, wq, dw, out)
    frac = assert_out_close(y, ref, out)
    log("  exact fraction", frac)


@pytest.mark.parametrize("m,n,k", [(40, 50, 256), (700, 1500, 256)])
def test_gemm_padded_output(m, n, k):
    xq = workloads.uniform_int8((m, k), seed=1, stream=4)
    wq = workloads.uniform_int8((n, k), seed=1, stream=5)
    dx = workloads.positive_scales(m, seed=2)
    dw = workloads.positive_scales(n, seed=3)
    big = torch.full((m, n + 13), -7.0, dtype=torch.float32, device=dev())
    y = big[:, :n]
    sq.sq_w8a8_linear(torch.from_numpy(xq).to(dev()), torch.from_numpy(dx).to(dev()), torch.from_numpy(wq).to(dev()),
                      torch.from_numpy(dw).to(dev()), out_dtype=torch.float32, y=y)
    assert np.array_equal(host(y), oracle.w8a8_linear(xq, dx, wq, dw, "f32"))
    assert np.all(host(big)[:, n:] == -7.0)


def test_gemm_deterministic():
    m, n, k = 300, 260, 2048
    xq = torch.from_numpy(workloads.uniform_int8((m, k), seed=9, stream=6)).to(dev())
    wq = torch.from_numpy(workloads.uniform_int8((n, k), seed=9, stream=7)).to(dev())
    first = host(sq.sq_w8a8_linear(xq, None, wq, None, out_dtype=torch.int32))
    for _ in range(3):
        assert np.array_equal(host(sq.sq_w8a8_linear(xq, None, wq, None, out_dtype=torch.int32)), first)


# --------------------------------------------------------------------------- fused run-time call
@pytest.mark.parametrize("m,k,n", [(1, 256, 64), (17, 512, 300), (200, 4096, 130)])
def test_linear_dyn_equals_two_calls(m, k, n):
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=m + k, dtype="bf16", calib_rows=64)
    s_ref = oracle.smoothing_factors(oracle.calibrate_absmax(c.x_calib), oracle.weight_row_absmax(c.w), 0.5)
    s = torch.from_numpy(s_ref).to(dev())
    _, wq, sw = sq.sq_smooth_fold_weights(to_dev(c.w, "bf16"), smooth=s, flags=sq.SMOOTH_GIVEN)
    x = to_dev(c.x, "bf16")
    y1 = sq.sq_w8a8_linear_dyn(x, s, wq, sw)
    xq, dx = sq.sq_quant_act_per_token(x, s)
    y2 = sq.sq_w8a8_linear(xq, dx, wq, sw)
    assert np.array_equal(bits16(y1), bits16(y2))
    wq_ref, sw_ref = oracle.quantize_weights_per_channel(oracle.fold_weights(c.w, s_ref))
    y_ref, _, _, _ = oracle.smoothquant_linear(c.x, s_ref, wq_ref, sw_ref, "bf16")
    assert_out_close(y1, y_ref, "bf16")


# --------------------------------------------------------------------------- LLM.int8()
@pytest.mark.parametrize("m,k,n,nout", [(64, 256, 96, 3), (130, 512, 200, 0), (257, 1024, 333, 9),
                                        (96, 256, 64, 256), (1030, 512, 1100, 5), (600, 256, 2000, 40)])
def test_int8_decomp_small(m, k, n, nout):
    log("decomp", m, k, n, nout)
    cfg = workloads.decomp_case(seed=m + n, m=m, k=k, n=n, n_outlier_cols=min(nout, k))
    thr = cfg.threshold if nout < k else 0.0
    x = cfg.x.copy()
    if nout >= k:
        x[x == 0] = 1.0  # every column strictly above 0
    xh, wh = to_dev(x, "f16"), to_dev(cfg.w, "f16")
    mask, idx, count = sq.sq_outlier_detect(xh, thr)
    m_ref = oracle.detect_outliers(x, thr)
    assert np.array_equal(host(mask).astype(bool), m_ref)
    cnt = int(host(count)[0])
    assert cnt == int(m_ref.sum()) and np.array_equal(host(idx)[:cnt], np.flatnonzero(m_ref))
    xq, dx = sq.sq_quant_act_rows_masked(xh, mask)
    xq_ref, dx_ref = oracle.quantize_rows_regular(x, m_ref)
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(dx), dx_ref)
    _, wq, sw = sq.sq_smooth_fold_weights(wh, flags=sq.SMOOTH_NONE)
    wq_ref, sw_ref = oracle.quantize_weights_per_channel(cfg.w)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(sw), sw_ref)
    y, n_out = sq.sq_int8_decomp_linear(xh, wq, sw, wh, thr)
    r = oracle.int8_decomp_linear(x, wq_ref, sw_ref, cfg.w, thr)
    assert int(host(n_out)[0]) == r["count"]
    got, ref = bits16(y), r["y"].view(np.uint16)
    bad = np.argwhere(got != ref)
    for i, j in bad[:8]:
        log("  mismatch", i, j, hex(got[i, j]), hex(ref[i, j]), "y_int", r["y_int"][i, j], "y_out", r["y_out"][i, j],
            "acc", r["acc"][i, j])
    assert len(bad) == 0, f"{len(bad)} mismatching outputs"


def test_int8_decomp_infinite_threshold_is_plain_int8():
    cfg = workloads.decomp_case(seed=4, m=100, k=512, n=150, n_outlier_cols=4)
    xh, wh = to_dev(cfg.x, "f16"), to_dev(cfg.w, "f16")
    _, wq, sw = sq.sq_smooth_fold_weights(wh, flags=sq.SMOOTH_NONE)
    y, n_out = sq.sq_int8_decomp_linear(xh, wq, sw, wh, float("inf"))
    xq, dx = sq.sq_quant_act_per_token(xh)
    y2 = sq.sq_w8a8_linear(xq, dx, wq, sw, out_dtype=torch.float16)
    assert int(host(n_out)[0]) == 0
    assert np.array_equal(bits16(y), bits16(y2))


@pytest.mark.parametrize("m,k,n,nout", [(300, 1024, 520, 6), (2048, 4096, 1024, 8), (17, 512, 64, 0)])
def test_int8_decomp_gemm_equals_linear(m, k, n, nout):
    """The GEMM half on its own, after detection and masked quantisation made by
    their own entry points, reproduces the one-call decomposition bit for bit."""
    log("decomp gemm", m, k, n, nout)
    cfg = workloads.decomp_case(seed=m + k, m=m, k=k, n=n, n_outlier_cols=nout)
    xh, wh = to_dev(cfg.x, "f16"), to_dev(cfg.w, "f16")
    _, wq, sw = sq.sq_smooth_fold_weights(wh, flags=sq.SMOOTH_NONE)
    y1, n1 = sq.sq_int8_decomp_linear(xh, wq, sw, wh, cfg.threshold)
    mask, idx, count = sq.sq_outlier_detect(xh, cfg.threshold)
    xq, dx = sq.sq_quant_act_rows_masked(xh, mask)
    y2 = sq.sq_int8_decomp_gemm(xq, dx, xh, wq, sw, wh, idx, count)
    assert int(host(n1)[0]) == int(host(count)[0])
    assert np.array_equal(bits16(y1), bits16(y2))
