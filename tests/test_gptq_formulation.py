"""The GPU's GPTQ formulation against the oracle, on the CPU.

The HIP sweep does not use the upper Cholesky factor of H^-1 as the GPTQ
paper does. It takes H = V V^T with V upper triangular (the Cholesky factor
of the index-reversed H, reversed back) and rounds
    z_j = w_j + sum_{i<j} (V_ij / V_jj) * (w_i - q_i * sw),
in blocks of 64 inputs with the later inputs updated by a GEMM. This test
writes that procedure in plain numpy, blocked the same way, and checks that
it yields the oracle's compensated weights and codes. So the reformulation
itself is checked independently of the GPU. It shares nothing with the HIP
code except the method.
"""
import numpy as np
import pytest

import oracle
import workloads

F32 = np.float32


def _v_form(wf, h, damp=0.01, block=64):
    w = np.asarray(wf, F32).astype(np.float64)
    k, n = w.shape
    h = np.array(h, np.float64, copy=True)
    dead = np.diag(h) == 0
    h[dead, dead] = 1.0
    w[dead, :] = 0.0
    sw = (np.abs(w.astype(F32)).max(axis=0).astype(F32) / F32(127)).astype(F32).astype(np.float64)
    h[np.diag_indices(k)] += damp * np.mean(np.diag(h))
    rev = h[::-1, ::-1]
    v = np.linalg.cholesky(rev)[::-1, ::-1]          # upper, H = V V^T
    assert np.allclose(np.tril(v, -1), 0) and np.allclose(v @ v.T, h, rtol=1e-10, atol=1e-10 * np.abs(h).max())
    c = v / np.diag(v)[None, :]                       # C_ij = V_ij / V_jj
    z = np.zeros((k, n))                              # running corrections
    zs = np.zeros((k, n))
    codes = np.zeros((k, n), np.int64)
    for j0 in range(0, k, block):
        d = np.zeros((block, n))
        for q in range(block):
            j = j0 + q
            zq = w[j] + z[j] + (c[j0:j, j] @ d[:q] if q else 0.0)
            zs[j] = zq
            with np.errstate(divide="ignore", invalid="ignore"):
                code = np.where(sw > 0, np.clip(np.rint(zq / sw), -127, 127), 0.0)
            codes[j] = code
            d[q] = w[j] - code * sw
        z[j0 + block:] += c[j0:j0 + block, j0 + block:].T @ d
    return codes.T, zs


@pytest.mark.parametrize("k,n,t,dead", [(128, 40, 300, ()), (256, 17, 512, (3, 130)), (192, 8, 64, ())])
def test_v_formulation_equals_oracle(k, n, t, dead):
    c = workloads.gptq_case(k, n, t, seed=k + t, dead=dead)
    s = oracle.smoothing_factors(oracle.calibrate_absmax(c.x_calib), oracle.weight_row_absmax(c.w), 0.5)
    wf = oracle.fold_weights(c.w, s)
    h = oracle.gptq_hessian(c.x_calib, s)
    wq_ref, sw_ref, z_ref = oracle.gptq_quantize(wf, h, trace=True)
    codes, z = _v_form(wf, h)
    scale = np.abs(z_ref).max()
    assert np.allclose(z, z_ref, rtol=0, atol=1e-9 * scale)
    assert np.array_equal(codes, wq_ref.astype(np.int64))
