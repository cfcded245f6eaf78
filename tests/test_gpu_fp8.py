"""Parity of the FP8 (E4M3) W8A8 variant.

The quantisers' codes and scales must equal the oracle's bit for bit. The
GEMM runs on the matrix cores' FP8 dot products, which are deterministic but
do not round their sums to nearest (measured on MI355X: within ~2^-12 of the
sum of |products| per 64-term instruction on codes of every magnitude). So
the output is compared with the oracle's exact product within a bound derived
from that: |y - y_exact| <= 2^-11 * d_i * sw_n * sum_k |x_ik w_nk| plus one
unit in the last place of the output type. Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import dev, host, log, padded, to_dev

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("w8a8_int8_quantization_amd")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,k", [(1, 64), (3, 448), (5, 4096), (64, 4096), (1030, 512), (300, 4160), (2, 14336),
                                 (2, 32768)])
def test_quant_act_fp8(dtype, m, k):
    log("fp8 act", dtype, m, k)
    c = workloads.random_linear_case(m=m, k=k, n=64, seed=m + k, dtype=dtype, calib_rows=8)
    x = c.x.copy()
    x[0, :3] = [0.0, -0.0, 1e-30] if dtype == "f32" else [0.0, -0.0, 0.0]
    xq, d = sq.sq_quant_act_fp8(to_dev(x, dtype))
    q_ref, d_ref = oracle.quantize_activations_fp8(x)
    assert np.array_equal(host(d).view(np.uint32), d_ref.view(np.uint32))
    rows = np.flatnonzero((host(xq) != q_ref).any(axis=1))
    assert rows.size == 0, f"codes differ in rows {rows[:5]}"


def test_quant_act_fp8_padded_and_zero_rows():
    c = workloads.random_linear_case(m=33, k=1024, n=64, seed=2, dtype="bf16", calib_rows=8)
    x = c.x.copy()
    x[5] = 0.0
    xq, d = sq.sq_quant_act_fp8(padded(x, "bf16", 1024 + 64))
    q_ref, d_ref = oracle.quantize_activations_fp8(x)
    assert np.array_equal(host(d), d_ref) and np.array_equal(host(xq), q_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("k,n", [(64, 64), (130, 192), (4096, 6144), (448, 4160)])
def test_quant_weights_fp8(dtype, k, n):
    log("fp8 weights", dtype, k, n)
    w = workloads.weights(k, n, seed=k + n, dtype=dtype)
    w[:, 3] = 0.0
    wq, sw = sq.sq_quant_weights_fp8(to_dev(w, dtype))
    wq_ref, sw_ref = oracle.quantize_weights_fp8(w)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
    assert np.array_equal(host(wq), wq_ref)


def _check_gemm(xq, d, wq, sw, out):
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out]
    y = sq.sq_fp8_linear(torch.from_numpy(xq).to(dev()), torch.from_numpy(d).to(dev()),
                         torch.from_numpy(wq).to(dev()), torch.from_numpy(sw).to(dev()), out_dtype=tdt)
    g = host(y.float()).astype(np.float64)
    a = oracle.e4m3_decode(xq).astype(np.float64)
    b = oracle.e4m3_decode(wq).astype(np.float64)
    exact = (a @ b.T) * d.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    mag = (np.abs(a) @ np.abs(b).T) * d.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    ulp_bits = {"bf16": 8, "f16": 11, "f32": 24}[out]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-38))) - (ulp_bits - 1))
    err = np.abs(g - exact)
    bound = 2.0 ** -11 * mag + ulp + 2.0 ** -22 * np.abs(exact)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3f}"
    ref = oracle.fp8_linear(xq, d, wq, sw, out)
    ref = ref.view(np.uint16) if out != "f32" else ref
    got_bits = host(y.view(torch.int16) if out != "f32" else y)
    same = float(np.mean(got_bits.view(ref.dtype) == ref)) if out != "f32" else float(np.mean(got_bits == ref))
    log("  max err/bound", float(np.max(err / bound)), "identical to the exact-sum oracle", same)
    return g, exact


@pytest.mark.parametrize("m,n,k", [(1, 1024, 4096), (17, 333, 1152), (64, 4096, 4096), (256, 512, 2048),
                                   (300, 192, 128), (2048, 6144, 4096)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_fp8_linear(m, n, k, out):
    log("fp8 gemm", m, n, k, out)
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=m + n + k, dtype="bf16", calib_rows=8)
    xq, d = oracle.quantize_activations_fp8(c.x)
    wq, sw = oracle.quantize_weights_fp8(c.w)
    g, exact = _check_gemm(xq, d, wq, sw, out)
    # the quantised product tracks the float product
    ref = c.x.astype(np.float64) @ c.w.astype(np.float64)
    assert np.linalg.norm(g - ref) <= 0.08 * np.linalg.norm(ref)


def test_fp8_linear_dyn_equals_two_calls():
    m, n, k = 96, 640, 2048
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=9, dtype="bf16", calib_rows=8)
    x = to_dev(c.x, "bf16")
    wq, sw = sq.sq_quant_weights_fp8(to_dev(c.w, "bf16"))
    xq, d = sq.sq_quant_act_fp8(x)
    y2 = sq.sq_fp8_linear(xq, d, wq, sw)
    nb = sq.raw["sq_fp8_linear_dyn_workspace_size"](m, n, k)
    ws = torch.full((nb,), 0x5C, dtype=torch.uint8, device=dev())
    y1 = sq.sq_fp8_linear_dyn(x, wq, sw, ws=ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# Prefill-sized problems (M >= 256, N >= 192, M N >= 2^20) run on the
# 256-row-tile pipeline (192- or 128-column tiles): ragged tiles in both
# directions, one and three k stages, every output type.
@pytest.mark.parametrize("m,n,k,out", [(1030, 1100, 1152, "f16"), (4096, 512, 128, "bf16"), (512, 2112, 384, "f32"),
                                       (777, 4000, 2176, "bf16"), (2048, 6144, 4096, "f16"), (1000, 6100, 1024, "bf16"),
                                       (2048, 4096, 4096, "f32")])
def test_fp8_linear_prefill_tiles(m, n, k, out):
    log("fp8 prefill gemm", m, n, k, out)
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=3 * m + n + k, dtype="bf16", calib_rows=8)
    xq, d = oracle.quantize_activations_fp8(c.x)
    wq, sw = oracle.quantize_weights_fp8(c.w)
    _check_gemm(xq, d, wq, sw, out)


# Shapes whose 256-column tiles fill the CUs at least once (and K is not
# split) run on four waves of 128 x 128 outputs: every output type, ragged
# tiles in both directions, a single k stage and a longer k.
@pytest.mark.parametrize("m,n,k,out", [(4096, 4096, 1024, "bf16"), (4352, 4160, 1280, "f32"), (4100, 4200, 128, "f16"),
                                       (4096, 4096, 3584, "bf16")])
def test_fp8_linear_prefill_four_wave_tiles(m, n, k, out):
    log("fp8 prefill gemm, four-wave tiles", m, n, k, out)
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=5 * m + n + k, dtype="bf16", calib_rows=8)
    xq, d = oracle.quantize_activations_fp8(c.x)
    wq, sw = oracle.quantize_weights_fp8(c.w)
    _check_gemm(xq, d, wq, sw, out)


def test_fp8_linear_prefill_random_codes():
    """Every finite E4M3 code in both operands (products from 2^-18 to 448^2),
    on the prefill pipeline."""
    m, n, k = 512, 2048, 1024
    rng = np.random.default_rng(77)
    xq = rng.integers(0, 256, size=(m, k), dtype=np.uint8)
    wq = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x00
    wq[(wq & 0x7F) == 0x7F] = 0x80
    d = rng.uniform(0.25, 4.0, size=m).astype(np.float32) * np.float32(2.0 ** -10)
    sw = rng.uniform(0.25, 4.0, size=n).astype(np.float32) * np.float32(2.0 ** -10)
    _check_gemm(xq, d, wq, sw, "f32")


@pytest.mark.parametrize("pad", [3, 8])
def test_fp8_linear_prefill_strided_output(pad):
    """Output rows with a pitch of n + pad elements: unaligned rows take the
    direct stores, aligned ones the staged rows; the padding is left alone."""
    m, n, k = 640, 1920, 512
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=pad, dtype="bf16", calib_rows=8)
    xq, d = oracle.quantize_activations_fp8(c.x)
    wq, sw = oracle.quantize_weights_fp8(c.w)
    big = torch.full((m, n + pad), -7.0, dtype=torch.bfloat16, device=dev())
    y = big[:, :n]
    sq.sq_fp8_linear(torch.from_numpy(xq).to(dev()), torch.from_numpy(d).to(dev()), torch.from_numpy(wq).to(dev()),
                     torch.from_numpy(sw).to(dev()), y=y)
    ref = sq.sq_fp8_linear(torch.from_numpy(xq).to(dev()), torch.from_numpy(d).to(dev()),
                           torch.from_numpy(wq).to(dev()), torch.from_numpy(sw).to(dev()))
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    assert bool((big[:, n:] == -7.0).all())
    _check_gemm(xq, d, wq, sw, "bf16")


# Decode shapes (M <= 64) run on the split-K decode kernel: one, two and four
# 16-token blocks, K split over up to 16 slices or not at all (N >= 12288,
# M > 16), ragged N.
@pytest.mark.parametrize("m,n,k,out", [(1, 4096, 4096, "bf16"), (16, 1000, 2048, "f16"), (32, 2112, 1152, "f32"),
                                       (64, 14336, 4096, "bf16"), (48, 200, 14336, "bf16"), (7, 64, 128, "f32")])
def test_fp8_linear_decode(m, n, k, out):
    log("fp8 decode gemm", m, n, k, out, "workspace bytes", sq.raw["sq_fp8_linear_workspace_size"](m, n, k))
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=5 * m + n + k, dtype="bf16", calib_rows=8)
    xq, d = oracle.quantize_activations_fp8(c.x)
    wq, sw = oracle.quantize_weights_fp8(c.w)
    _check_gemm(xq, d, wq, sw, out)


def test_fp8_linear_decode_workspace_reuse():
    """The split-K counters are left at zero: the same workspace serves the
    next call, at this shape and at a smaller one, with identical results."""
    m, n, k = 8, 1024, 4096
    assert sq.raw["sq_fp8_linear_workspace_size"](m, n, k) > 0
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=21, dtype="bf16", calib_rows=8)
    xq, d = oracle.quantize_activations_fp8(c.x)
    wq, sw = oracle.quantize_weights_fp8(c.w)
    args = [torch.from_numpy(a).to(dev()) for a in (xq, d, wq, sw)]
    ws = sq.fp8_linear_workspace(m, n, k, dev())
    y1 = sq.sq_fp8_linear(*args, ws=ws)
    y2 = sq.sq_fp8_linear(*args, ws=ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert int(ws[:256].view(torch.int32)[: (n + 63) // 64].abs().sum()) == 0
    y3 = sq.sq_fp8_linear(args[0][:3], args[1][:3], *args[2:], ws=ws)
    assert torch.equal(y3.view(torch.int16), y1[:3].view(torch.int16))
    _check_gemm(xq, d, wq, sw, "bf16")


@pytest.mark.parametrize("m", [1, 40])
def test_fp8_linear_dyn_decode_garbage_workspace(m):
    """The one-call path clears the split-K counters itself: a workspace full
    of garbage gives the result of the two separate calls."""
    n, k = 768, 2048
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=m, dtype="bf16", calib_rows=8)
    x = to_dev(c.x, "bf16")
    wq, sw = sq.sq_quant_weights_fp8(to_dev(c.w, "bf16"))
    xq, d = sq.sq_quant_act_fp8(x)
    y2 = sq.sq_fp8_linear(xq, d, wq, sw)
    nb = sq.raw["sq_fp8_linear_dyn_workspace_size"](m, n, k)
    assert nb > sq.raw["sq_fp8_linear_workspace_size"](m, n, k) > 0
    ws = torch.full((nb,), 0xA7, dtype=torch.uint8, device=dev())
    y1 = sq.sq_fp8_linear_dyn(x, wq, sw, ws=ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    y1b = sq.sq_fp8_linear_dyn(x, wq, sw, ws=ws)
    assert torch.equal(y1b.view(torch.int16), y2.view(torch.int16))
