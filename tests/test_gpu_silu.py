"""Parity of the fused gated activation SiLU(gate) * up + smoothing + per-token
quantisation (the down projection's input).

Codes and row scales must equal the oracle's bit for bit: both evaluate SiLU
with the same fixed binary32 exponential, one IEEE operation per step. Gate
values out to +-120 cover SiLU's saturated ends and the exponential's
overflow and underflow. Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_out_close, dev, host, log, padded, to_dev

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("w8a8_int8_quantization_amd")


def _check(gate, up, s, ld=0):
    g = padded(gate, "bf16", ld) if ld else to_dev(gate, "bf16")
    u = padded(up, "bf16", ld) if ld else to_dev(up, "bf16")
    sd = None if s is None else torch.from_numpy(s).to(dev())
    xq, d = sq.sq_silu_mul_quant(g, u, sd)
    q_ref, d_ref = oracle.silu_mul_quantize(gate, up, s)
    got_d = host(d)
    bad = np.flatnonzero(got_d.view(np.uint32) != d_ref.view(np.uint32))
    assert bad.size == 0, f"row scales differ in {bad.size} rows, first {bad[:5]}"
    rows = np.flatnonzero((host(xq) != q_ref).any(axis=1))
    assert rows.size == 0, f"codes differ in {rows.size} rows, first {rows[:5]}"


# one vector per thread and less; several; decode rows (1024 threads); rows
# beyond the grid; the down projection's 14336; the longest rows
SHAPES = [(1, 64), (3, 448), (5, 4096), (64, 14336), (1030, 512), (300, 4160), (7, 14336), (2, 32768)]


@pytest.mark.parametrize("m,k", SHAPES)
@pytest.mark.parametrize("smooth", ["none", "calibrated", "spread"])
def test_silu_mul_quant(m, k, smooth):
    log("silu", m, k, smooth)
    c = workloads.gate_up_case(m, k, seed=m + k, calib_rows=64)
    if smooth == "none":
        s = None
    elif smooth == "calibrated":
        a = oracle.calibrate_absmax(oracle.gated_activation(c.gate_calib, c.up_calib))
        w = workloads.weights(k, 64, seed=k, dtype="bf16")
        s = oracle.smoothing_factors(a, oracle.weight_row_absmax(w), 0.5)
    else:  # factors over every binade, past the fast range too
        s = workloads.spread_scales(k, seed=k, lo_exp=-24, hi_exp=24)
    _check(c.gate, c.up, s)


def test_silu_mul_quant_exp_edges():
    """Gate values across the exponential's whole range, one row per decade."""
    k = 512
    rows = []
    for lo, hi in [(-0.5, 0.5), (-20, 20), (-90, -80), (-130, -100), (80, 90), (100, 130), (-15, -14)]:
        rows.append(np.linspace(lo, hi, k))
    gate = workloads._as_dtype(np.array(rows, np.float32), "bf16")
    up = workloads._as_dtype(np.tile(np.linspace(-3, 3, k), (len(rows), 1)).astype(np.float32), "bf16")
    _check(gate, up, None)
    _check(gate, up, workloads.spread_scales(k, seed=7, lo_exp=-6, hi_exp=6))
    z = np.zeros((2, k), np.float32)
    _check(z, z, None)   # all-zero rows: scale 0, codes 0
    # bf16 values around the tabulated range's ends (|g| near 2^-25 and 128), both signs, and zeros
    fields = np.concatenate([np.arange(96, 106), np.arange(130, 140)])
    vals = [((f << 7) | mant) for f in fields for mant in (0, 1, 63, 127)]
    bits = np.array(vals + [v | 0x8000 for v in vals] + [0, 0x8000], np.uint32)
    g = (np.resize(bits, (2, k)) << 16).view(np.float32)
    _check(g, np.full((2, k), 1.5, np.float32), None)


def test_silu_mul_quant_padded():
    c = workloads.gate_up_case(40, 1024, seed=3)
    _check(c.gate, c.up, workloads.spread_scales(1024, seed=3, lo_exp=-3, hi_exp=3), ld=1024 + 64)


def test_silu_mul_quant_full_down_prefill():
    """The down projection's prefill input, 8192 x 14336 (every row checked
    against the oracle on a sample of 512 rows, all rows on the GPU)."""
    m, k = 8192, 14336
    c = workloads.gate_up_case(m, k, seed=11, calib_rows=128)
    a = oracle.calibrate_absmax(oracle.gated_activation(c.gate_calib, c.up_calib))
    w = workloads.weights(k, 64, seed=11, dtype="bf16")
    s = oracle.smoothing_factors(a, oracle.weight_row_absmax(w), 0.5)
    log("silu full", m, k)
    xq, d = sq.sq_silu_mul_quant(to_dev(c.gate, "bf16"), to_dev(c.up, "bf16"), torch.from_numpy(s).to(dev()))
    idx = np.random.default_rng(0).choice(m, 512, replace=False)
    q_ref, d_ref = oracle.silu_mul_quantize(c.gate[idx], c.up[idx], s)
    assert np.array_equal(host(d)[idx].view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(host(xq)[idx], q_ref)


@pytest.mark.parametrize("m,n,k", [(1, 1024, 14336), (16, 333, 2048), (64, 4096, 14336), (256, 512, 4096)])
def test_silu_mul_w8a8_linear(m, n, k):
    """Gated activation + quantisation + GEMM in one call equals the oracle's
    layer within 1 ulp of bf16 on a workspace that was never initialised."""
    log("silu linear", m, n, k)
    c = workloads.gate_up_case(m, k, seed=m + n + k, calib_rows=64)
    w = workloads.weights(k, n, seed=m + n + k, dtype="bf16")
    a = oracle.calibrate_absmax(oracle.gated_activation(c.gate_calib, c.up_calib))
    s = oracle.smoothing_factors(a, oracle.weight_row_absmax(w), 0.5)
    wq_ref, sw_ref = oracle.quantize_weights_per_channel(oracle.fold_weights(w, s))
    xq_ref, dx_ref = oracle.silu_mul_quantize(c.gate, c.up, s)
    y_ref = oracle.w8a8_linear(xq_ref, dx_ref, wq_ref, sw_ref, "bf16")
    nb = sq.raw["sq_silu_mul_w8a8_linear_workspace_size"](m, n, k)
    ws = torch.full((nb,), 0x77, dtype=torch.uint8, device=dev())
    g, u = to_dev(c.gate, "bf16"), to_dev(c.up, "bf16")
    sd, wq, sw = torch.from_numpy(s).to(dev()), torch.from_numpy(wq_ref).to(dev()), torch.from_numpy(sw_ref).to(dev())
    for _ in range(2):
        y = sq.sq_silu_mul_w8a8_linear(g, u, sd, wq, sw, ws=ws)
        frac = assert_out_close(y, y_ref, "bf16")
    log("  exact fraction", frac)
