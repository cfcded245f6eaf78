"""Edge cases on the GPU: empty inputs through every run-time call, and the
int8 prefill kernel at the largest K the int32 accumulator allows.

Zero-sized calls must return without error and enqueue nothing. At
K = 133,120 (the largest multiple of 128 with 127^2 K < 2^31) rows of +-127
give accumulators of +-2,147,092,480, within 2^31 - 1 = 2,147,483,647; the
expected values are the closed form 127^2 K s_i t_n.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("w8a8_int8_quantization_amd")


def _empty(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device=dev())


def test_zero_sized_calls():
    k, n = 256, 192
    wq = torch.zeros((n, k), dtype=torch.int8, device=dev())
    sw = torch.ones(n, dtype=torch.float32, device=dev())
    x0 = _empty(0, k)
    xq, d = sq.sq_quant_act_per_token(x0, None)
    assert xq.shape == (0, k) and d.shape == (0,)
    y = sq.sq_w8a8_linear(xq, d, wq, sw)
    assert y.shape == (0, n)
    assert sq.sq_w8a8_linear_dyn(x0, None, wq, sw).shape == (0, n)
    gain = torch.ones(k, dtype=torch.float32, device=dev())
    xq, d = sq.sq_rmsnorm_quant(x0, gain, 1e-6)
    assert xq.shape == (0, k)
    xq, d = sq.sq_silu_mul_quant(x0, x0, None)
    assert xq.shape == (0, k)
    xq8, d8 = sq.sq_quant_act_fp8(x0)
    wq8 = torch.zeros((n, k), dtype=torch.uint8, device=dev())
    assert sq.sq_fp8_linear(xq8, d8, wq8, sw).shape == (0, n)
    assert sq.sq_fp8_linear_dyn(x0, wq8, sw).shape == (0, n)
    h = sq.sq_gptq_hessian(x0)
    torch.cuda.synchronize()
    assert float(h.abs().sum()) == 0.0
    # no output channels
    wq0 = torch.zeros((0, k), dtype=torch.int8, device=dev())
    x = torch.ones((4, k), dtype=torch.bfloat16, device=dev())
    assert sq.sq_w8a8_linear_dyn(x, None, wq0, sw[:0]).shape == (4, 0)
    torch.cuda.synchronize()


def test_prefill_kernel_at_max_k():
    """1024 x 1024 outputs (the 256-row-tile kernel) at K = 133,120: every
    accumulator is +-127^2 K or 0, exactly."""
    m, n, k = 1024, 1024, 133120
    assert 127 * 127 * k < 2 ** 31
    rng = np.random.default_rng(4)
    si = rng.choice([-1, 0, 1], size=m).astype(np.int8)
    tn = rng.choice([-1, 1], size=n).astype(np.int8)
    xq = (torch.from_numpy(si).to(dev())[:, None] * 127).expand(m, k).contiguous()
    wq = (torch.from_numpy(tn).to(dev())[:, None] * 127).expand(n, k).contiguous()
    log("max-K prefill GEMM", m, n, k)
    acc = host(sq.sq_w8a8_linear(xq, None, wq, None, out_dtype=torch.int32))
    ref = 127 * 127 * k * (si.astype(np.int64)[:, None] * tn.astype(np.int64)[None, :])
    assert np.array_equal(acc.astype(np.int64), ref)
