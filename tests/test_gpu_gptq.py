"""Parity of GPTQ weight rounding on the GPU against the oracle.

The Hessian is compared entry by entry (exactly, where the sums are exact in
binary64; otherwise within binary64 rounding). The quantisation sweep is
compared code by code. The GPU uses an equivalent formulation (the
Cholesky factor of H instead of that of its inverse, blocked updates), so its
binary64 roundings differ from the oracle's in the last bits. A code may
therefore differ only where the oracle's quotient lies within 1e-9 of a
half-integer; after such a tie the rest of that channel follows a different
but equally valid path and is not compared. Scales are bit-exact. Every call
goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import dev, host, log, to_dev

pytestmark = pytest.mark.gpu

sq = pytest.importorskip("w8a8_int8_quantization_amd")

TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _smoothing(c):
    a = oracle.calibrate_absmax(c.x_calib)
    return oracle.smoothing_factors(a, oracle.weight_row_absmax(c.w), 0.5)


def _compare(wq_gpu, sw_gpu, wq_ref, sw_ref, z_ref):
    """Codes equal to the oracle's up to each channel's first tie (see the module notes)."""
    assert np.array_equal(sw_gpu.view(np.uint32), sw_ref.view(np.uint32)), "scales differ"
    diff = wq_gpu != wq_ref
    bad_channels = np.flatnonzero(diff.any(axis=1))
    for n in bad_channels:
        j = int(np.flatnonzero(diff[n])[0])
        r = z_ref[j, n] / np.float64(sw_ref[n])
        assert abs(abs(r - np.floor(r)) - 0.5) < 1e-9, \
            f"channel {n}: code {j} differs ({wq_gpu[n, j]} vs {wq_ref[n, j]}) away from a tie (z/sw = {r!r})"
    log("  channels with a tie:", len(bad_channels), "of", wq_ref.shape[0])
    assert len(bad_channels) <= max(1, wq_ref.shape[0] // 100)


def _gpu_gptq(c, s, damp=0.01):
    x = to_dev(c.x_calib, c.dtype)
    st = torch.from_numpy(s).to(dev()) if s is not None else None
    h = sq.sq_gptq_hessian(x, st)
    wq, sw = sq.sq_gptq_quantize(h, to_dev(c.w, c.dtype), st, damp=damp)
    torch.cuda.synchronize()
    return host(h), host(wq), host(sw)


def test_gptq_hessian_exact_sums():
    """Eighths and power-of-two smoothing factors: every product and sum is
    exact in binary64, so H equals the oracle's bit for bit; two calls over
    halves of the rows add up to the same H."""
    rng = np.random.default_rng(3)
    t, k = 96, 256
    x = (rng.integers(-64, 65, size=(t, k)) / 8.0).astype(np.float32)
    s = np.exp2(rng.integers(-3, 4, size=k)).astype(np.float32)
    ref = oracle.gptq_hessian(x, s)
    xd, sd = to_dev(x, "f32"), torch.from_numpy(s).to(dev())
    h = host(sq.sq_gptq_hessian(xd, sd))
    assert np.array_equal(h, ref)
    h2 = sq.sq_gptq_hessian(xd[: t // 2], sd)
    h2 = host(sq.sq_gptq_hessian(xd[t // 2:], sd, h=h2))
    assert np.array_equal(h2, ref)


@pytest.mark.parametrize("dtype,t,k", [("bf16", 1000, 384), ("f16", 77, 128), ("f32", 300, 512)])
def test_gptq_hessian(dtype, t, k):
    c = workloads.gptq_case(k, 64, t, seed=k + t, dtype=dtype)
    s = _smoothing(c)
    ref = oracle.gptq_hessian(c.x_calib, s)
    h = host(sq.sq_gptq_hessian(to_dev(c.x_calib, dtype), torch.from_numpy(s).to(dev())))
    assert np.array_equal(h, h.T)
    scale = np.sqrt(np.outer(np.diag(ref), np.diag(ref)))
    assert np.all(np.abs(h - ref) <= 1e-13 * t * scale)


@pytest.mark.parametrize("k,n,t,dtype,dead,smooth", [
    (128, 64, 256, "bf16", (), True),
    (256, 333, 512, "bf16", (5, 200), True),
    (512, 200, 1024, "f16", (), False),
    (1024, 130, 2048, "f32", (0, 1023), True),
    (128, 1, 64, "bf16", (), True),
    (2176, 999, 700, "bf16", (17, 2175), True),
])
def test_gptq_quantize(k, n, t, dtype, dead, smooth):
    log("gptq", k, n, t, dtype, dead, smooth)
    c = workloads.gptq_case(k, n, t, seed=k + n, dtype=dtype, dead=dead)
    s = _smoothing(c) if smooth else None
    wf = oracle.fold_weights(c.w, s) if s is not None else c.w
    wq_ref, sw_ref, z_ref = oracle.gptq_quantize(wf, oracle.gptq_hessian(c.x_calib, s), trace=True)
    _, wq, sw = _gpu_gptq(c, s)
    _compare(wq, sw, wq_ref, sw_ref, z_ref)
    for j in dead:
        assert np.all(wq[:, j] == 0)


def test_gptq_deterministic_and_better_than_rtn():
    """Two runs give identical codes; on the calibration inputs the layer's
    output error is far below that of round-to-nearest (the library's own
    per-channel RTN with the same smoothing)."""
    c = workloads.gptq_case(512, 384, 2048, seed=11)
    s = _smoothing(c)
    _, wq1, sw1 = _gpu_gptq(c, s)
    _, wq2, sw2 = _gpu_gptq(c, s)
    assert np.array_equal(wq1, wq2) and np.array_equal(sw1, sw2)
    _, rq, rs = sq.sq_smooth_fold_weights(to_dev(c.w, "bf16"), smooth=torch.from_numpy(s).to(dev()),
                                          flags=sq.SMOOTH_GIVEN)
    rq, rs = host(rq), host(rs)
    wf = oracle.fold_weights(c.w, s).astype(np.float64)
    xh = oracle.smooth_activations(c.x_calib, s).astype(np.float64)
    e_g = np.linalg.norm(xh @ (wq1.T.astype(np.float64) * sw1.astype(np.float64) - wf))
    e_r = np.linalg.norm(xh @ (rq.T.astype(np.float64) * rs.astype(np.float64) - wf))
    log("  output error GPTQ / RTN:", e_g / e_r)
    assert e_g < 0.7 * e_r


def test_gptq_full_size_sampled_channels():
    """The QKV layer at full size (K 4096, N 6144, 4096 calibration rows):
    the oracle, from its own Hessian, sweeps 8 sampled output channels (the
    channels are independent given H) and must agree with the GPU's codes."""
    k, n, t = 4096, 6144, 4096
    c = workloads.gptq_case(k, n, t, seed=0)
    s = _smoothing(c)
    _, wq, sw = _gpu_gptq(c, s)
    cols = np.array([0, 1, 777, 2048, 3001, 4095, 5000, n - 1])
    h_ref = oracle.gptq_hessian(c.x_calib, s)
    wf = oracle.fold_weights(c.w, s)
    wq_ref, sw_ref, z_ref = oracle.gptq_quantize(wf[:, cols], h_ref, trace=True)
    _compare(wq[cols], sw[cols], wq_ref, sw_ref, z_ref)
    assert np.all(np.abs(wq.astype(np.int64)) <= 127) and np.all(sw > 0)

