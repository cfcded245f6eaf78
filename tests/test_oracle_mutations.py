"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

Every mutant replaces one oracle function by a copy with one mistake (a dropped
term, a wrong sign or exponent, a transposed operand, a wrong rounding). The
test passes only if at least one pin in ``oracle_pins.ALL_PINS`` fails on the
mutant, which shows the pins constrain every part of the oracle.
"""
import importlib

import numpy as np
import pytest

import oracle
from oracle import llm_int8 as o_int8
from oracle import numerics as o_num
from oracle import smoothquant as o_sq
from tests import oracle_pins

# the submodule (the package attribute of the same name is the function rmsnorm)
o_rms = importlib.import_module("oracle.rmsnorm")
o_silu = importlib.import_module("oracle.silu")
o_fp8 = importlib.import_module("oracle.fp8")
o_gptq = importlib.import_module("oracle.gptq")

F32 = np.float32


def _smooth_swapped(a, w, alpha):
    a64, w64 = np.asarray(a, np.float64), np.asarray(w, np.float64)
    ok = (a64 > 0) & (w64 > 0)
    with np.errstate(all="ignore"):
        s = np.power(a64, 1 - alpha) / np.power(w64, alpha)
    return np.where(ok, s, 1.0).astype(F32)


def _smooth_product(a, w, alpha):
    a64, w64 = np.asarray(a, np.float64), np.asarray(w, np.float64)
    ok = (a64 > 0) & (w64 > 0)
    with np.errstate(all="ignore"):
        s = np.power(a64, alpha) * np.power(w64, 1 - alpha)
    return np.where(ok, s, 1.0).astype(F32)


def _smooth_zero_not_one(a, w, alpha):
    a64, w64 = np.asarray(a, np.float64), np.asarray(w, np.float64)
    with np.errstate(all="ignore"):
        s = np.power(a64, alpha) / np.power(w64, 1 - alpha)
    return np.nan_to_num(s, nan=0.0, posinf=0.0).astype(F32)


def _fold_divides(w, s):
    return (np.asarray(w, F32) / np.asarray(s, F32)[:, None]).astype(F32)


def _smooth_act_multiplies(x, s):
    x = np.asarray(x, F32)
    return x.copy() if s is None else (x * np.asarray(s, F32)[None, :]).astype(F32)


def _quant_w_per_row(wf):
    wf = np.asarray(wf, F32)
    rowmax = np.abs(wf).max(axis=1).astype(F32)
    scale = (rowmax / F32(127)).astype(F32)
    with np.errstate(all="ignore"):
        q = np.clip(np.rint((wf / scale[:, None]).astype(F32)), -127, 127)
    q = np.where(scale[:, None] > 0, q, 0)
    return np.ascontiguousarray(q.T.astype(np.int8)), scale[: wf.shape[1]] if wf.shape[1] <= wf.shape[0] \
        else np.resize(scale, wf.shape[1])


def _quant_w_qmax128(wf):
    wf = np.asarray(wf, F32)
    colmax = np.abs(wf).max(axis=0).astype(F32)
    scale = (colmax / F32(128)).astype(F32)
    with np.errstate(all="ignore"):
        q = np.clip(np.rint((wf / scale[None, :]).astype(F32)), -127, 127)
    q = np.where(scale[None, :] > 0, q, 0)
    return np.ascontiguousarray(q.T.astype(np.int8)), scale


def _quant_w_no_transpose(wf):
    wq, sw = o_sq.__dict__["_orig_quantize_weights_per_channel"](wf)
    return np.ascontiguousarray(wq.T).reshape(wq.shape), sw


def _quant_act_trunc(x, s=None):
    xh = o_sq.smooth_activations(x, s)
    scale = (np.abs(xh).max(axis=1).astype(F32) / F32(127)).astype(F32)
    with np.errstate(all="ignore"):
        q = np.clip(np.trunc((xh / scale[:, None]).astype(F32)), -127, 127)
    return np.where(scale[:, None] > 0, q, 0).astype(np.int8), scale


def _quant_act_half_away(x, s=None):
    xh = o_sq.smooth_activations(x, s)
    scale = (np.abs(xh).max(axis=1).astype(F32) / F32(127)).astype(F32)
    with np.errstate(all="ignore"):
        r = (xh / scale[:, None]).astype(F32)
    q = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127)
    return np.where(scale[:, None] > 0, q, 0).astype(np.int8), scale


def _quant_act_per_tensor(x, s=None):
    xh = o_sq.smooth_activations(x, s)
    scale = np.full(xh.shape[0], F32(np.abs(xh).max() / F32(127)), F32)
    with np.errstate(all="ignore"):
        q = np.clip(np.rint((xh / scale[:, None]).astype(F32)), -127, 127)
    return np.where(scale[:, None] > 0, q, 0).astype(np.int8), scale


def _quant_act_ignores_s(x, s=None):
    return o_sq.__dict__["_orig_quantize_activations"](x, None)


def _gemm_reversed_k(xq, wq):
    return o_sq.__dict__["_orig_int8_matmul"](xq, np.ascontiguousarray(np.asarray(wq)[:, ::-1]))


def _gemm_no_overflow_check(xq, wq):
    return (np.asarray(xq, np.float64) @ np.asarray(wq, np.float64).T).astype(np.int64).astype(np.int32)


def _dequant_drops_w_scale(acc, x_scale, w_scale, out="bf16"):
    y = (np.asarray(acc, np.int32).astype(F32) * np.asarray(x_scale, F32)[:, None]).astype(F32)
    return o_num.round_to(y, out)


def _dequant_swaps_scales(acc, x_scale, w_scale, out="bf16"):
    acc = np.asarray(acc, np.int32)
    xs = np.resize(np.asarray(w_scale, F32), acc.shape[0])
    ws = np.resize(np.asarray(x_scale, F32), acc.shape[1])
    y = (acc.astype(F32) * xs[:, None]).astype(F32)
    return o_num.round_to((y * ws[None, :]).astype(F32), out)


def _bf16_truncates(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _calib_signed_max(x_rows, prior=None):
    x = np.asarray(x_rows, F32)
    a = x.max(axis=0)
    return (np.maximum(a, prior) if prior is not None else a).astype(F32)


def _calib_ignores_prior(x_rows, prior=None):
    return np.abs(np.asarray(x_rows, F32)).max(axis=0).astype(F32)


def _row_absmax_by_column(w):
    w = np.abs(np.asarray(w, F32))
    return np.resize(w.max(axis=0), w.shape[0]).astype(F32)


def _detect_ge(x, threshold):
    return np.abs(np.asarray(x, F32)).max(axis=0) >= F32(threshold)


def _rows_regular_all_cols(x, mask):
    xf = np.asarray(x, F32)
    scale = (np.abs(xf).max(axis=1).astype(F32) / F32(127)).astype(F32)
    with np.errstate(all="ignore"):
        q = np.clip(np.rint((np.where(mask[None, :], 0, xf) / scale[:, None]).astype(F32)), -127, 127)
    return np.where(scale[:, None] > 0, q, 0).astype(np.int8), scale


def _outlier_product_drops_last(x, w16, mask):
    m = mask.copy()
    idx = np.flatnonzero(m)
    if len(idx):
        m[idx[-1]] = False
    return o_int8.__dict__["_orig_fp16_outlier_product"](x, w16, m)


def _outlier_product_wrong_row(x, w16, mask):
    return o_int8.__dict__["_orig_fp16_outlier_product"](x, np.roll(np.asarray(w16), 1, axis=0), mask)


def _rms_chain(x, eps, reduce):
    x = np.asarray(x, F32)
    out = np.zeros(x.shape[0], F32)
    for i in range(x.shape[0]):
        v = reduce(x[i].astype(np.float64), float(F32(eps)))
        with np.errstate(all="ignore"):
            inv = F32(1.0 / v) if v > 0 else F32(0)
        out[i] = inv if np.isfinite(inv) else 0
    return out


def _rms_sum_not_mean(x, eps=0.0):
    return _rms_chain(x, eps, lambda r, e: np.sqrt(np.sum(r * r) + e))


def _rms_eps_outside_root(x, eps=0.0):
    return _rms_chain(x, eps, lambda r, e: np.sqrt(np.mean(r * r)) + e)


def _rms_drops_last(x, eps=0.0):
    return _rms_chain(x, eps, lambda r, e: np.sqrt(np.sum(r[:-1] ** 2) / len(r) + e))


def _rms_mean_abs(x, eps=0.0):
    return _rms_chain(x, eps, lambda r, e: np.mean(np.abs(r)) + e)


def _gain_divides(normalized, gain):
    return (np.asarray(normalized, F32) / np.asarray(gain, F32)[None, :]).astype(F32)


def _fold_gain_multiplies(gamma, s):
    g = np.asarray(gamma, F32)
    return g.copy() if s is None else (g * np.asarray(s, F32)).astype(F32)


def _rmsnorm_drops_gain(x, gain, eps=0.0):
    x = np.asarray(x, F32)
    return (x * o_rms.rms_inverse(x, eps)[:, None]).astype(F32)


def _rmsnorm_gain_before_norm(x, gain, eps=0.0):
    xg = o_rms.apply_gain(x, gain)
    return (xg * o_rms.rms_inverse(xg, eps)[:, None]).astype(F32)


def _exp_variant(drop_top=False, drop_lo=False):
    def f(t):
        t = np.asarray(t, dtype=F32)
        coefs = o_silu.EXP_COEF[1:] if drop_top else o_silu.EXP_COEF
        with np.errstate(all="ignore"):
            k = np.clip(np.rint((t * o_silu.INV_LN2).astype(F32)), -256, 256).astype(F32)
            r = (t - (k * o_silu.LN2_HI).astype(F32)).astype(F32)
            if not drop_lo:
                r = (r - (k * o_silu.LN2_LO).astype(F32)).astype(F32)
            p = np.full_like(r, coefs[0])
            for c in coefs[1:]:
                p = ((p * r).astype(F32) + c).astype(F32)
            e = np.ldexp(p, k.astype(np.int32)).astype(F32)
        e = np.where(t > o_silu.T_HI, F32(np.inf), e)
        return np.where(t < o_silu.T_LO, F32(0.0), e).astype(F32)
    return f


def _silu_wrong_sign(z):
    z = np.asarray(z, dtype=F32)
    with np.errstate(all="ignore"):
        return (z * (F32(1.0) / (F32(1.0) + o_silu.exp32(z)).astype(F32))).astype(F32)


def _gated_swapped(gate, up):
    return o_num.round_bf16((o_silu.silu32(np.asarray(up, F32)) * np.asarray(gate, F32)).astype(F32))


def _gated_no_bf16(gate, up):
    return (o_silu.silu32(np.asarray(gate, F32)) * np.asarray(up, F32)).astype(F32)


def _e4m3_round_half_up(v):
    v = np.asarray(v, dtype=np.float64)
    vals = o_fp8.e4m3_values()
    pos = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    a = np.minimum(np.abs(v), 448.0)
    idx = np.searchsorted(pos, a, side="right") - 1
    idx = np.clip(idx, 0, len(pos) - 2)
    lo, hi = pos[idx], pos[idx + 1]
    r = np.where(a - lo >= hi - a, hi, lo)
    r = np.where(a >= pos[-1], pos[-1], r)
    out = np.array([int(np.flatnonzero(vals == x)[0]) for x in r], np.uint8)
    return np.where(np.signbit(v) & (r > 0), out | 0x80, out).astype(np.uint8)


def _e4m3_truncate(v):
    v = np.asarray(v, dtype=np.float64)
    vals = o_fp8.e4m3_values()
    pos = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    a = np.minimum(np.abs(v), 448.0)
    r = pos[np.clip(np.searchsorted(pos, a, side="right") - 1, 0, len(pos) - 1)]
    out = np.array([int(np.flatnonzero(vals == x)[0]) for x in r], np.uint8)
    return np.where(np.signbit(v) & (r > 0), out | 0x80, out).astype(np.uint8)


def _fp8_act_scale_127(x):
    x = np.asarray(x, F32)
    d = (np.abs(x).max(axis=1).astype(F32) / F32(127)).astype(F32)
    with np.errstate(all="ignore"):
        v = (x / d[:, None]).astype(F32)
    return o_fp8.e4m3_encode(np.where(d[:, None] > 0, v, F32(0))), d


def _fp8_w_scale_per_row(w):
    w = np.asarray(w, F32)
    rowmax = np.abs(w).max(axis=1).astype(F32)
    s = (rowmax / F32(448)).astype(F32)
    with np.errstate(all="ignore"):
        v = (w / s[:, None]).astype(F32)
    codes = o_fp8.e4m3_encode(np.where(s[:, None] > 0, v, F32(0)))
    return np.ascontiguousarray(codes.T), np.resize(s, w.shape[1]).astype(F32)


def _gptq_variant(sign=1.0, divide=True, factor="upper_inverse", damp=True, reach=None, half_away=False,
                  error_from_original=False):
    """gptq_quantize with one mistake: the update's sign, the division by U_jj,
    the factor used (lower Cholesky of H, or of H^-1), no damping, errors
    passed only ``reach`` weights on, ties rounded away from zero, or the
    error measured against the original rather than the compensated weight."""
    def f(w_folded, h, damp_frac=0.01, trace=False):
        w = np.asarray(w_folded, dtype=F32).astype(np.float64)
        w0 = w.copy()
        k, n = w.shape
        h = np.array(h, dtype=np.float64, copy=True)
        dead = np.diag(h) == 0
        h[dead, dead] = 1.0
        w[dead, :] = 0.0
        sw = (np.abs(w.astype(F32)).max(axis=0).astype(F32) / F32(127)).astype(F32)
        sw64 = sw.astype(np.float64)
        if damp:
            h[np.diag_indices(k)] += damp_frac * np.mean(np.diag(h))
        if factor == "upper_inverse":
            u = np.linalg.cholesky(np.linalg.inv(h)).T
        elif factor == "lower_inverse":
            u = np.linalg.cholesky(np.linalg.inv(h))
        else:
            u = np.linalg.cholesky(h).T
        codes = np.zeros((k, n), np.int8)
        z = np.zeros((k, n))
        for j in range(k):
            wj = w[j].copy()
            z[j] = wj
            with np.errstate(all="ignore"):
                r = wj / sw64
                q = np.sign(r) * np.floor(np.abs(r) + 0.5) if half_away else np.rint(r)
                q = np.where(sw64 > 0, np.clip(q, -127, 127), 0.0)
            codes[j] = q.astype(np.int8)
            base = w0[j] if error_from_original else wj
            err = (base - q * sw64) / (u[j, j] if divide else 1.0)
            end = k if reach is None else min(k, j + 1 + reach)
            w[j + 1:end] -= sign * np.outer(u[j, j + 1:end], err)
        out = (np.ascontiguousarray(codes.T), sw)
        return out + (z,) if trace else out
    return f


def _gptq_hessian_unsmoothed(x_cal, s=None):
    x = np.asarray(x_cal, F32).astype(np.float64)
    return x.T @ x


def _gptq_hessian_times_s(x_cal, s=None):
    x = np.asarray(x_cal, F32)
    if s is not None:
        x = (x * np.asarray(s, F32)[None, :]).astype(F32)
    x = x.astype(np.float64)
    return x.T @ x


def _gptq_hessian_rows(x_cal, s=None):
    x = o_sq.smooth_activations(x_cal, s).astype(np.float64)
    return x @ x.T


MUTANTS = {
    "s_exponents_swapped": (o_sq, "smoothing_factors", _smooth_swapped),
    "s_product_not_quotient": (o_sq, "smoothing_factors", _smooth_product),
    "s_zero_channel_not_one": (o_sq, "smoothing_factors", _smooth_zero_not_one),
    "fold_divides_weight": (o_sq, "fold_weights", _fold_divides),
    "activation_multiplied_by_s": (o_sq, "smooth_activations", _smooth_act_multiplies),
    "weight_scale_per_row": (o_sq, "quantize_weights_per_channel", _quant_w_per_row),
    "weight_qmax_128": (o_sq, "quantize_weights_per_channel", _quant_w_qmax128),
    "weight_not_transposed": (o_sq, "quantize_weights_per_channel", _quant_w_no_transpose),
    "act_truncates": (o_sq, "quantize_activations", _quant_act_trunc),
    "act_round_half_away": (o_sq, "quantize_activations", _quant_act_half_away),
    "act_per_tensor_scale": (o_sq, "quantize_activations", _quant_act_per_tensor),
    "act_ignores_smoothing": (o_sq, "quantize_activations", _quant_act_ignores_s),
    "gemm_wrong_k_index": (o_sq, "int8_matmul", _gemm_reversed_k),
    "gemm_no_overflow_guard": (o_sq, "int8_matmul", _gemm_no_overflow_check),
    "dequant_drops_weight_scale": (o_sq, "dequantize", _dequant_drops_w_scale),
    "dequant_swaps_scales": (o_sq, "dequantize", _dequant_swaps_scales),
    "bf16_truncates": (o_num, "f32_to_bf16_bits", _bf16_truncates),
    "calib_drops_abs": (o_sq, "calibrate_absmax", _calib_signed_max),
    "calib_ignores_running_max": (o_sq, "calibrate_absmax", _calib_ignores_prior),
    "weight_rowmax_wrong_axis": (o_sq, "weight_row_absmax", _row_absmax_by_column),
    "detect_not_strict": (o_int8, "detect_outliers", _detect_ge),
    "row_scale_includes_outliers": (o_int8, "quantize_rows_regular", _rows_regular_all_cols),
    "fp16_slice_drops_column": (o_int8, "fp16_outlier_product", _outlier_product_drops_last),
    "fp16_slice_wrong_weight_row": (o_int8, "fp16_outlier_product", _outlier_product_wrong_row),
    "rms_sum_not_mean": (o_rms, "rms_inverse", _rms_sum_not_mean),
    "rms_eps_outside_root": (o_rms, "rms_inverse", _rms_eps_outside_root),
    "rms_drops_last_channel": (o_rms, "rms_inverse", _rms_drops_last),
    "rms_mean_abs_not_root_mean_square": (o_rms, "rms_inverse", _rms_mean_abs),
    "norm_gain_divides": (o_rms, "apply_gain", _gain_divides),
    "norm_fold_multiplies": (o_rms, "fold_norm_gain", _fold_gain_multiplies),
    "rmsnorm_drops_gain": (o_rms, "rmsnorm", _rmsnorm_drops_gain),
    "rmsnorm_gain_before_norm": (o_rms, "rmsnorm", _rmsnorm_gain_before_norm),
    "exp_drops_top_taylor_term": (o_silu, "exp32", _exp_variant(drop_top=True)),
    "exp_drops_low_ln2_part": (o_silu, "exp32", _exp_variant(drop_lo=True)),
    "silu_exponent_sign": (o_silu, "silu32", _silu_wrong_sign),
    "gated_silu_on_up": (o_silu, "gated_activation", _gated_swapped),
    "gated_no_bf16_rounding": (o_silu, "gated_activation", _gated_no_bf16),
    "e4m3_round_half_up": (o_fp8, "e4m3_encode", _e4m3_round_half_up),
    "e4m3_truncates": (o_fp8, "e4m3_encode", _e4m3_truncate),
    "fp8_act_scale_127": (o_fp8, "quantize_activations_fp8", _fp8_act_scale_127),
    "fp8_weight_scale_per_row": (o_fp8, "quantize_weights_fp8", _fp8_w_scale_per_row),
    "gptq_update_sign": (o_gptq, "gptq_quantize", _gptq_variant(sign=-1.0)),
    "gptq_no_division_by_ujj": (o_gptq, "gptq_quantize", _gptq_variant(divide=False)),
    "gptq_cholesky_of_h": (o_gptq, "gptq_quantize", _gptq_variant(factor="upper_h")),
    "gptq_lower_factor": (o_gptq, "gptq_quantize", _gptq_variant(factor="lower_inverse")),
    "gptq_no_damping": (o_gptq, "gptq_quantize", _gptq_variant(damp=False)),
    "gptq_error_to_next_only": (o_gptq, "gptq_quantize", _gptq_variant(reach=1)),
    "gptq_round_half_away": (o_gptq, "gptq_quantize", _gptq_variant(half_away=True)),
    "gptq_error_from_original_weight": (o_gptq, "gptq_quantize", _gptq_variant(error_from_original=True)),
    "gptq_hessian_unsmoothed": (o_gptq, "gptq_hessian", _gptq_hessian_unsmoothed),
    "gptq_hessian_multiplies_s": (o_gptq, "gptq_hessian", _gptq_hessian_times_s),
    "gptq_hessian_over_tokens": (o_gptq, "gptq_hessian", _gptq_hessian_rows),
}


def _plant(monkeypatch, module, name, fn):
    monkeypatch.setitem(module.__dict__, "_orig_" + name, getattr(module, name))
    monkeypatch.setattr(module, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)
    # functions re-exported through another submodule's namespace
    for mod in (o_sq, o_int8, o_num, o_rms, o_silu, o_fp8, o_gptq):
        if mod is not module and name in mod.__dict__:
            monkeypatch.setitem(mod.__dict__, name, fn)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches(mutant, monkeypatch):
    module, name, fn = MUTANTS[mutant]
    _plant(monkeypatch, module, name, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle)
        except Exception as e:  # AssertionError, or a shape error the mistake causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {mutant}"
