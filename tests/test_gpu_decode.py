"""Parity of the decode-shaped GEMM (M <= 64 tokens, K a multiple of 128, and
65..256 tokens where the decode kernel is chosen, one grid layer per 64).

These shapes run the split-K decode kernel (its unrolled form up to 16
tokens, its LDS-ring form from 17): per-slice int32 partial tiles in the
workspace, ticket counters, the last workgroup of a tile reducing. The
int32 accumulators must equal the oracle's exact integer product; dequantised
outputs must be within 1 ulp of the oracle. Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_out_close, bits16, dev, host, log, to_dev

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("w8a8_int8_quantization_amd")

# (n, k): one step; ragged N (N % 4 != 0 and N % 64 != 0); slices whose step
# count does not divide among the 4 waves; both 8B decode projections; K near
# the int32 limit (hundreds of slices).
NK = [(64, 128), (99, 256), (301, 1152), (130, 8192), (4096, 14336), (14336, 4096), (64, 133120)]
MS = [1, 5, 16, 17, 33, 64]
# more than one 64-token block (ragged last block)
MS_WIDE = [65, 100, 128, 200, 256]


def _dev_i8(a):
    return torch.from_numpy(a).to(dev())


@pytest.mark.parametrize("n,k", NK)
@pytest.mark.parametrize("m", MS)
def test_decode_int32_exact(m, n, k):
    if k > 20000 and m not in (1, 64):
        pytest.skip("the longest K runs at the smallest and largest M only")
    log("decode i32", m, n, k, "ws", sq.raw["sq_w8a8_linear_workspace_size"](m, n, k))
    xq = workloads.uniform_int8((m, k), seed=m * 7 + n + k, stream=10)
    wq = workloads.uniform_int8((n, k), seed=m * 7 + n + k, stream=11)
    acc = sq.sq_w8a8_linear(_dev_i8(xq), None, _dev_i8(wq), None, out_dtype=torch.int32)
    assert np.array_equal(host(acc), oracle.int8_matmul(xq, wq))


@pytest.mark.parametrize("n,k", [(4096, 14336), (14336, 4096), (301, 1152), (64, 128)])
@pytest.mark.parametrize("m", MS_WIDE)
def test_decode_int32_exact_wide(m, n, k):
    """Token blocks beyond the first (the shapes the decode kernel takes
    above 64 tokens, and the others through whichever kernel they route to)."""
    log("decode i32 wide", m, n, k, "ws", sq.raw["sq_w8a8_linear_workspace_size"](m, n, k))
    xq = workloads.uniform_int8((m, k), seed=m * 3 + n + k, stream=14)
    wq = workloads.uniform_int8((n, k), seed=m * 3 + n + k, stream=15)
    acc = sq.sq_w8a8_linear(_dev_i8(xq), None, _dev_i8(wq), None, out_dtype=torch.int32)
    assert np.array_equal(host(acc), oracle.int8_matmul(xq, wq))


# K slices longer than the unrolled kernel's 32 steps: more column tiles than
# the split's ticket counters, so K is not split (the 17..256-token ring form
# loops over the whole K; fewer tokens route to the tiled kernels); 70B-style
# layers (28672 x 8192), a ragged 257-tile layer, and two 64-token layers.
@pytest.mark.parametrize("m,n,k", [(1, 28672, 8192), (8, 28672, 8192), (17, 16448, 8192), (32, 28672, 8192),
                                   (64, 16448, 8192), (96, 14336, 14336)])
def test_decode_long_slices_exact(m, n, k):
    log("decode long slices", m, n, k, "ws", sq.raw["sq_w8a8_linear_workspace_size"](m, n, k))
    xq = workloads.uniform_int8((m, k), seed=m + n + k, stream=16)
    wq = workloads.uniform_int8((n, k), seed=m + n + k, stream=17)
    acc = sq.sq_w8a8_linear(_dev_i8(xq), None, _dev_i8(wq), None, out_dtype=torch.int32)
    assert np.array_equal(host(acc), oracle.int8_matmul(xq, wq))


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("m,n,k", [(1, 4096, 14336), (8, 301, 1152), (32, 14336, 4096), (64, 99, 256), (100, 4096, 14336), (256, 14336, 4096)])
def test_decode_dequant(out, m, n, k):
    log("decode dequant", out, m, n, k)
    xq = workloads.uniform_int8((m, k), seed=m + n, stream=12)
    wq = workloads.uniform_int8((n, k), seed=m + n, stream=13)
    dx = workloads.positive_scales(m, seed=m, stream=2)
    dw = workloads.positive_scales(n, seed=n, stream=3) * np.float32(1e-3)
    y = sq.sq_w8a8_linear(_dev_i8(xq), torch.from_numpy(dx).to(dev()), _dev_i8(wq), torch.from_numpy(dw).to(dev()),
                          out_dtype={"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out])
    frac = assert_out_close(y, oracle.w8a8_linear(xq, dx, wq, dw, out), out)
    log("  exact fraction", frac)


@pytest.mark.parametrize("m", [24, 128])
def test_decode_workspace_reuse(m):
    """sq_w8a8_linear: a workspace zero-filled once stays usable (the kernel
    restores its ticket counters, one per 64 columns and 64-token block).
    sq_w8a8_linear_dyn: a workspace full of garbage works (the quantisation
    launch clears the counters)."""
    n, k = 4096, 14336
    nb = sq.raw["sq_w8a8_linear_workspace_size"](m, n, k)
    assert nb > 0
    xq = workloads.uniform_int8((m, k), seed=5, stream=14)
    wq = workloads.uniform_int8((n, k), seed=5, stream=15)
    ref = oracle.int8_matmul(xq, wq)
    ws = sq.linear_workspace(m, n, k, dev())
    x_d, w_d = _dev_i8(xq), _dev_i8(wq)
    for _ in range(3):
        acc = sq.sq_w8a8_linear(x_d, None, w_d, None, out_dtype=torch.int32, ws=ws)
        assert np.array_equal(host(acc), ref)
        assert not host(ws[:4 * ((n + 63) // 64) * ((m + 63) // 64)]).any(), "ticket counters not restored"
    c = workloads.random_linear_case(m=m, k=k, n=n, seed=3, dtype="bf16", calib_rows=64)
    s_ref = oracle.smoothing_factors(oracle.calibrate_absmax(c.x_calib), oracle.weight_row_absmax(c.w), 0.5)
    s = torch.from_numpy(s_ref).to(dev())
    _, wq2, sw2 = sq.sq_smooth_fold_weights(to_dev(c.w, "bf16"), smooth=s, flags=sq.SMOOTH_GIVEN)
    x = to_dev(c.x, "bf16")
    nbd = sq.raw["sq_w8a8_linear_dyn_workspace_size"](m, n, k)
    wsd = torch.full((nbd,), 0x5A, dtype=torch.uint8, device=dev())
    first = bits16(sq.sq_w8a8_linear_dyn(x, s, wq2, sw2, ws=wsd))
    for _ in range(2):
        assert np.array_equal(bits16(sq.sq_w8a8_linear_dyn(x, s, wq2, sw2, ws=wsd)), first)
    wq_ref, sw_ref = oracle.quantize_weights_per_channel(oracle.fold_weights(c.w, s_ref))
    y_ref, _, _, _ = oracle.smoothquant_linear(c.x, s_ref, wq_ref, sw_ref, "bf16")
    assert_out_close(torch.from_numpy(first.view(np.int16)).view(torch.bfloat16), y_ref, "bf16")


def test_decode_workspace_validation():
    m, n, k = 4, 4096, 14336
    nb = sq.raw["sq_w8a8_linear_workspace_size"](m, n, k)
    xq = torch.zeros((m, k), dtype=torch.int8, device=dev())
    wq = torch.zeros((n, k), dtype=torch.int8, device=dev())
    y = torch.empty((m, n), dtype=torch.int32, device=dev())
    small = torch.empty(nb - 1, dtype=torch.uint8, device=dev())
    st = sq.raw["sq_w8a8_linear"](xq.data_ptr(), None, wq.data_ptr(), None, m, n, k, y.data_ptr(), 3, n,
                                  small.data_ptr(), nb - 1, None)
    assert st == 6  # SQ_ERR_WORKSPACE
    st = sq.raw["sq_w8a8_linear"](xq.data_ptr(), None, wq.data_ptr(), None, m, n, k, y.data_ptr(), 3, n,
                                  None, 0, None)
    assert st == 6


# One token: sq_w8a8_linear_dyn runs the quantisation inside the one-token
# product (one launch) for layers at least 2048 wide, and quantisation +
# split-K decode GEMM otherwise. (dtype, n, k): the 8B up and down
# projections, ragged N, the longest rows the fused path takes (16384 bf16 /
# fp16 values with 16 waves, 8192 binary32 with 8), one-step K, the narrowest
# fused layer, and layers on the two-launch path (narrower, or binary32 rows
# of 16384). Up to K = 8192 a workgroup runs 1, 2, 4 or 8 tiles of 8 rows
# (the grid nearest 448 workgroups): 2048 / 4096 columns one tile, 5000 /
# 6150 two, 9600 / 12290 / 14336 four, 28672 / 28680 eight, ragged last
# workgroups among them; beyond K = 8192 (16 waves) as many tiles as keep the
# grid within 256 workgroups: 2056 / 4096 columns two, 12300 eight.
ONE_TOKEN = [("bf16", 14336, 4096), ("bf16", 12300, 16384), ("f16", 12290, 1152), ("f32", 14336, 8192),
             ("f32", 12288, 128), ("bf16", 28672, 256), ("bf16", 4096, 14336), ("f16", 300, 1152),
             ("f32", 2050, 16384), ("bf16", 2048, 128), ("f16", 6150, 5120), ("bf16", 28680, 4096),
             ("f32", 9600, 4096), ("f16", 5000, 8192), ("f16", 2056, 9216)]


def _one_token_case(dtype, n, k, seed, smooth_kind):
    c = workloads.random_linear_case(m=1, k=k, n=n, seed=seed, dtype=dtype, calib_rows=8)
    x = to_dev(c.x, dtype)
    if smooth_kind == "none":
        s = None
    elif smooth_kind == "fast":
        s = torch.from_numpy(workloads.spread_scales(k, seed=seed, lo_exp=-6, hi_exp=6)).to(dev())
    else:  # factors outside the quotients' fast range: IEEE division throughout
        s = torch.from_numpy(workloads.spread_scales(k, seed=seed, lo_exp=-30, hi_exp=30)).to(dev())
    _, wq, sw = sq.sq_smooth_fold_weights(to_dev(c.w, dtype), flags=sq.SMOOTH_NONE)
    return x, s, wq, sw


@pytest.mark.parametrize("smooth_kind", ["fast", "wide", "none"])
@pytest.mark.parametrize("dtype,n,k", ONE_TOKEN)
def test_one_token_fused_equals_two_calls(dtype, n, k, smooth_kind):
    """Row scale, codes and outputs of the fused one-token step are those of
    the quantisation kernel followed by the GEMM, bit for bit."""
    log("one token fused", dtype, n, k, smooth_kind)
    x, s, wq, sw = _one_token_case(dtype, n, k, seed=n + k, smooth_kind=smooth_kind)
    for out in (torch.bfloat16, torch.float32, torch.float16):
        y1 = sq.sq_w8a8_linear_dyn(x, s, wq, sw, out_dtype=out)
        xq, dx = sq.sq_quant_act_per_token(x, s)
        y2 = sq.sq_w8a8_linear(xq, dx, wq, sw, out_dtype=out)
        iv = torch.int32 if out == torch.float32 else torch.int16
        assert torch.equal(y1.view(iv), y2.view(iv)), out


def test_one_token_fused_zero_row_and_oracle():
    """A zero token gives zero outputs; a real one matches the oracle."""
    k, n = 4096, 14336
    c = workloads.linear_case("decode_up", m=1)
    s_ref = oracle.smoothing_factors(oracle.calibrate_absmax(c.x_calib), oracle.weight_row_absmax(c.w), c.alpha)
    s = torch.from_numpy(s_ref).to(dev())
    _, wq, sw = sq.sq_smooth_fold_weights(to_dev(c.w, "bf16"), smooth=s, flags=sq.SMOOTH_GIVEN)
    y0 = sq.sq_w8a8_linear_dyn(torch.zeros((1, k), dtype=torch.bfloat16, device=dev()), s, wq, sw)
    assert int((bits16(y0) != 0).sum()) == 0
    y = sq.sq_w8a8_linear_dyn(to_dev(c.x, "bf16"), s, wq, sw)
    wq_ref, sw_ref = oracle.quantize_weights_per_channel(oracle.fold_weights(c.w, s_ref))
    y_ref, _, _, _ = oracle.smoothquant_linear(c.x, s_ref, wq_ref, sw_ref, "bf16")
    assert_out_close(y, y_ref, "bf16")


@pytest.mark.parametrize("dtype,n,k", [("bf16", 14336, 4096), ("bf16", 4096, 14336), ("f32", 2050, 16384)])
def test_one_token_fused_workspace_reuse(dtype, n, k):
    """The one-launch step publishes the row's codes and scale through the
    workspace: a workspace full of garbage, one reused call after call (with
    different inputs and layers of different K), and the library's static
    scratch all give the two-call result, bit for bit."""
    log("one token workspace reuse", dtype, n, k)
    nb = sq.raw["sq_w8a8_linear_dyn_workspace_size"](1, n, 16384)
    ws = torch.randint(0, 256, (nb,), dtype=torch.uint8, device=dev())
    layers = [_one_token_case(dtype, n, k, seed=11 + i, smooth_kind="fast") for i in range(3)]
    layers.append(_one_token_case(dtype, n, 4096 if k != 4096 else 8192, seed=23, smooth_kind="fast"))
    for rep in range(2):
        for x, s, wq, sw in layers:
            xq, dx = sq.sq_quant_act_per_token(x, s)
            y2 = sq.sq_w8a8_linear(xq, dx, wq, sw, out_dtype=torch.bfloat16)
            y1 = sq.sq_w8a8_linear_dyn(x, s, wq, sw, out_dtype=torch.bfloat16, ws=ws)
            y3 = sq.sq_w8a8_linear_dyn_static(x, s, wq, sw, out_dtype=torch.bfloat16)
            assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), rep
            assert torch.equal(y3.view(torch.int16), y2.view(torch.int16)), rep
