"""The five workloads at their full sizes, through the same calls the benchmark times.

Calibration statistics, smoothing factors, Wq, w_scale, Xq and x_scale are
compared in full; the GEMM output on every row for the small configurations
and, for the large ones, on a stratified sample of rows (all columns) that the
oracle computes row by row: one row for every position within the 256-row
tiles (each from a seeded random tile) plus the last row, so every row slot
of the kernels' tiles and the ragged tail are checked at full size.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_out_close, bits16, dev, host, log, to_dev, ulp_diff32

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("w8a8_int8_quantization_amd")

ROW_SAMPLE = 256  # rows per tile of the prefill kernel


def _stratified_rows(m: int, seed: int) -> np.ndarray:
    """One row for each residue mod ROW_SAMPLE (in a random tile), plus m - 1."""
    rng = np.random.default_rng(seed)
    rows = [r + ROW_SAMPLE * int(rng.integers(0, (m - r + ROW_SAMPLE - 1) // ROW_SAMPLE))
            for r in range(min(ROW_SAMPLE, m))]
    return np.unique(np.array(rows + [m - 1], dtype=np.int64))


def _run_linear(c, sample_rows):
    log("config", c.name, c.m, c.k, c.n, "alpha", c.alpha)
    dt = c.x_dtype
    xc, x, w = to_dev(c.x_calib, dt), to_dev(c.x, dt), to_dev(c.w, c.w_dtype)
    a = torch.zeros(c.k, dtype=torch.float32, device=dev())
    sq.sq_calibrate_absmax(xc, a)
    a_ref = oracle.calibrate_absmax(c.x_calib)
    assert np.array_equal(host(a), a_ref), "calibration absmax"
    s_gpu, _, _ = sq.sq_smooth_fold_weights(w, c.alpha, absmax=a)
    s_ref = oracle.smoothing_factors(a_ref, oracle.weight_row_absmax(c.w), c.alpha)
    d = ulp_diff32(host(s_gpu), s_ref)
    assert d.max() <= 1, "smoothing factor beyond 1 ulp"
    log("  s exact fraction", float((d == 0).mean()))
    s = torch.from_numpy(s_ref).to(dev())
    _, wq, sw = sq.sq_smooth_fold_weights(w, smooth=s, flags=sq.SMOOTH_GIVEN)
    wq_ref, sw_ref = oracle.quantize_weights_per_channel(oracle.fold_weights(c.w, s_ref))
    assert np.array_equal(host(sw), sw_ref), "w_scale"
    assert np.array_equal(host(wq), wq_ref), "Wq"
    out = {"f32": torch.float32, "bf16": torch.bfloat16}[c.y_dtype]
    y = sq.sq_w8a8_linear_dyn(x, s, wq, sw, out_dtype=out)
    xq, dx = sq.sq_quant_act_per_token(x, s)
    xq_ref, dx_ref = oracle.quantize_activations(c.x, s_ref)
    assert np.array_equal(host(dx), dx_ref), "x_scale"
    assert np.array_equal(host(xq), xq_ref), "Xq"
    rows = np.arange(c.m) if not sample_rows else _stratified_rows(c.m, c.m + c.n)
    acc_ref = oracle.int8_matmul(xq_ref[rows], wq_ref)
    y_ref = oracle.dequantize(acc_ref, dx_ref[rows], sw_ref, c.y_dtype)
    acc = sq.sq_w8a8_linear(xq, dx, wq, sw, out_dtype=torch.int32)
    assert np.array_equal(host(acc)[rows], acc_ref), "int32 accumulators"
    frac = assert_out_close(y[torch.from_numpy(rows).to(dev())], y_ref, c.y_dtype)
    log("  output exact fraction", frac)


def test_tiny_fp32():
    _run_linear(workloads.linear_case("tiny"), sample_rows=0)


def test_qkv_prefill():
    _run_linear(workloads.linear_case("qkv_prefill"), sample_rows=ROW_SAMPLE)


@pytest.mark.parametrize("alpha", [0.5, 0.8])
def test_gateup_prefill(alpha):
    _run_linear(workloads.linear_case("gateup_prefill", alpha=alpha), sample_rows=ROW_SAMPLE)


@pytest.mark.parametrize("alpha", [0.5, 0.8])
def test_down_prefill(alpha):
    _run_linear(workloads.linear_case("down_prefill", alpha=alpha), sample_rows=ROW_SAMPLE)


@pytest.mark.parametrize("name", ["decode_up", "decode_down"])
@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_decode(name, m):
    _run_linear(workloads.linear_case(name, m=m), sample_rows=0)


def test_llm_int8_full():
    cfg = workloads.decomp_case()
    log("config llm_int8", cfg.m, cfg.k, cfg.n)
    xh, wh = to_dev(cfg.x, "f16"), to_dev(cfg.w, "f16")
    _, wq, sw = sq.sq_smooth_fold_weights(wh, flags=sq.SMOOTH_NONE)
    y, n_out = sq.sq_int8_decomp_linear(xh, wq, sw, wh, cfg.threshold)
    wq_ref, sw_ref = oracle.quantize_weights_per_channel(cfg.w)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(sw), sw_ref)
    mask_ref = oracle.detect_outliers(cfg.x, cfg.threshold)
    assert int(host(n_out)[0]) == int(mask_ref.sum()) == len(cfg.channels)
    mask, idx, count = sq.sq_outlier_detect(xh, cfg.threshold)
    assert np.array_equal(host(mask).astype(bool), mask_ref)
    xq, dx = sq.sq_quant_act_rows_masked(xh, mask)
    xq_ref, dx_ref = oracle.quantize_rows_regular(cfg.x, mask_ref)
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(dx), dx_ref)
    rows = _stratified_rows(cfg.m, 5)
    r = oracle.int8_decomp_linear(cfg.x[rows], wq_ref, sw_ref, cfg.w, cfg.threshold, mask=mask_ref)
    assert np.array_equal(bits16(y)[rows], r["y"].view(np.uint16))
