"""CPU oracle of the SmoothQuant W8A8 linear layer (test infrastructure only).

Each function writes one step of the method out as its plain definition, in
numpy, with every binary32 operation spelled as a single numpy float32
operation (IEEE-754 round-to-nearest-even), so a reader can check it against
the pages by eye. The pages cited:

* "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
  LLM Quantization" (called "the W8A8 post" below), sections "How the Model Was
  Compressed", "Why Naive Weight Quantization Doesn't Work, and How GPTQ Fixes
  It", "Why Activation Quantization Is Hard, and How SmoothQuant Fixes It",
  "Where the outlier actually comes from", "How the smoothing factor is
  computed" and "Performance After Quantization" (Inter-Token Latency).
* "How does SmoothQuant int8 LLM calibration work ..." (called "the calibration
  Q&A"), section "The Technical Workflow for Int8 Quantization Deployment".
* The LLM.int8() page, section "The architecture: every piece explained".

Readings taken where the pages are silent or garbled (each one is listed with
its reason in the design notes):

* The smoothing-factor equation itself did not survive text extraction; its
  symbols are defined in "How the smoothing factor is computed". The formula
  used is s_j = A_j^alpha / W_j^(1-alpha) with A_j, W_j absolute maxima,
  evaluated in binary64 and rounded once to binary32. A zero A_j or W_j gives
  s_j = 1 (no smoothing on a channel with no signal).
* "round" is round-half-to-even; the int8 range is symmetric, [-127, 127].
* The smoothed weight stays binary32 (no bf16 rounding in between), because
  fold and quantisation are one step here.
* The dequantisation order is ((float)acc * x_scale_i) * w_scale_n in binary32.
* A zero scale gives a zero quantised row / column.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .numerics import round_to

QMAX = 127
F32 = np.float32


def _f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32)


# --------------------------------------------------------------------------
# Calibration: per-input-channel activation absmax
# --------------------------------------------------------------------------
def calibrate_absmax(x_rows: np.ndarray, prior: Optional[np.ndarray] = None) -> np.ndarray:
    """A_j = largest |activation| seen in input channel j over the calibration rows.

    The W8A8 post, "How the smoothing factor is computed": A_j is the largest
    activation observed in channel j across the calibration samples; the
    calibration Q&A, "The Technical Workflow ...": the statistic is the maximum
    absolute value per channel. ``prior`` carries the running maximum over
    earlier calibration batches.
    """
    x = _f32(x_rows)
    a = np.abs(x).max(axis=0) if x.shape[0] else np.zeros(x.shape[1], F32)
    if prior is not None:
        a = np.maximum(a, _f32(prior))
    return a.astype(F32)


def weight_row_absmax(w: np.ndarray) -> np.ndarray:
    """W_j = largest |weight| in row j of the receiving layer's W [K x N].

    The W8A8 post, "How the smoothing factor is computed": W_j belongs to the
    weight row that matches input channel j.
    """
    return np.abs(_f32(w)).max(axis=1).astype(F32)


# --------------------------------------------------------------------------
# Smoothing factor
# --------------------------------------------------------------------------
def smoothing_factors(a: np.ndarray, w_rowmax: np.ndarray, alpha: float) -> np.ndarray:
    """s_j = A_j^alpha / W_j^(1 - alpha), binary64 powers, rounded once to binary32.

    The W8A8 post, "How the smoothing factor is computed" (alpha moves the
    quantisation difficulty from activations to weights; large s on outlier
    channels, s near 1 elsewhere); the calibration Q&A gives alpha in [0, 1].
    Channels with A_j = 0 or W_j = 0 get s_j = 1.
    """
    if not (0.0 <= alpha <= 1.0):
        raise ValueError("alpha must lie in [0, 1]")
    a64 = _f32(a).astype(np.float64)
    w64 = _f32(w_rowmax).astype(np.float64)
    ok = (a64 > 0) & (w64 > 0)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        s64 = np.power(a64, float(alpha)) / np.power(w64, 1.0 - float(alpha))
    return np.where(ok, s64, 1.0).astype(F32)


# --------------------------------------------------------------------------
# Fold + per-output-channel weight quantisation
# --------------------------------------------------------------------------
def fold_weights(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W'_jn = s_j * W_jn in binary32: row j of W is scaled up by s_j.

    The W8A8 post, "Where the outlier actually comes from" (the next layer's
    weights are scaled up on the matching input channel) and "How the
    smoothing factor is computed" (row j times s_j).
    """
    return (_f32(s)[:, None] * _f32(w)).astype(F32)


def quantize_weights_per_channel(w_folded: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 RTN with one scale per output channel (weight column).

    The W8A8 post, "How the Model Was Compressed": scale = max|column| / 127,
    q = round(w / scale); "Why Naive Weight Quantization ...": one scale per
    column (channel). Returns (Wq [N x K] int8, the transpose of the
    quantised W, and w_scale [N] binary32).
    """
    wf = _f32(w_folded)
    colmax = np.abs(wf).max(axis=0).astype(F32)            # [N]
    scale = (colmax / F32(QMAX)).astype(F32)               # fl32(max / 127)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (wf / scale[None, :]).astype(F32)          # fl32(w / scale)
    q = np.clip(np.rint(ratio), -QMAX, QMAX)
    q = np.where(scale[None, :] > 0, q, 0.0)
    return np.ascontiguousarray(q.T.astype(np.int8)), scale


def smooth_fold_quantize(a: np.ndarray, w: np.ndarray, alpha: float,
                         s: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Offline weight preparation: s (unless given), fold, quantise.

    Returns (s [K] binary32, Wq [N x K] int8, w_scale [N] binary32).
    """
    if s is None:
        s = smoothing_factors(a, weight_row_absmax(w), alpha)
    wq, sw = quantize_weights_per_channel(fold_weights(w, s))
    return _f32(s), wq, sw


# --------------------------------------------------------------------------
# Per-token dynamic activation quantisation
# --------------------------------------------------------------------------
def smooth_activations(x: np.ndarray, s: Optional[np.ndarray]) -> np.ndarray:
    """x_hat_ij = x_ij / s_j in binary32 (x itself when there is no smoothing).

    The W8A8 post, "How the smoothing factor is computed": the activation side
    is divided by s (there through the norm gain; here applied to x directly).
    """
    x = _f32(x)
    if s is None:
        return x.copy()
    return (x / _f32(s)[None, :]).astype(F32)


def quantize_activations(x: np.ndarray, s: Optional[np.ndarray] = None
                         ) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token symmetric int8: one scale per row over all channels.

    The W8A8 post, "How the Model Was Compressed" (a single scale per token,
    computed at run time over all of its channels) and "Why Activation
    Quantization Is Hard ..." (scale = max|x| / 127, q = round(x / scale)).
    Returns (Xq [M x K] int8, x_scale [M] binary32).
    """
    xh = smooth_activations(x, s)
    rowmax = np.abs(xh).max(axis=1).astype(F32) if xh.shape[1] else np.zeros(xh.shape[0], F32)
    scale = (rowmax / F32(QMAX)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (xh / scale[:, None]).astype(F32)
    q = np.clip(np.rint(ratio), -QMAX, QMAX)
    q = np.where(scale[:, None] > 0, q, 0.0)
    return q.astype(np.int8), scale


# --------------------------------------------------------------------------
# int8 x int8 -> int32 GEMM and the dequantisation epilogue
# --------------------------------------------------------------------------
def int8_matmul(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc_in = sum_k Xq_ik * Wq_nk, exact.

    The LLM.int8() page, "The architecture ...": the int8 operands are
    multiplied with an int32 accumulator. Computed as a binary64 product of
    integer-valued operands: every partial sum is an integer below 2^53, so the
    result is exact whatever order the library sums in.
    """
    xq = np.asarray(xq, dtype=np.int8)
    wq = np.asarray(wq, dtype=np.int8)
    if xq.shape[1] != wq.shape[1]:
        raise ValueError("inner dimensions differ")
    acc = xq.astype(np.float64) @ wq.astype(np.float64).T
    if acc.size and np.abs(acc).max() >= 2.0 ** 31:
        raise OverflowError("int32 accumulator overflow")
    return acc.astype(np.int64).astype(np.int32)


def dequantize(acc: np.ndarray, x_scale: np.ndarray, w_scale: np.ndarray,
               out: str = "bf16") -> np.ndarray:
    """y_in = ((float)acc_in * x_scale_i) * w_scale_n in binary32, then the output type.

    The LLM.int8() page, "The architecture ...": the accumulator is scaled by
    the row scale times the column scale; the W8A8 post, "Inter-Token
    Latency": the result is converted back to bf16. ``out`` is 'f32', 'bf16'
    (returned as uint16 bit patterns) or 'f16'.
    """
    a32 = np.asarray(acc, dtype=np.int32).astype(F32)      # int -> binary32, RNE
    y = (a32 * _f32(x_scale)[:, None]).astype(F32)
    y = (y * _f32(w_scale)[None, :]).astype(F32)
    return round_to(y, out)


def w8a8_linear(xq, x_scale, wq, w_scale, out: str = "bf16") -> np.ndarray:
    """int8 GEMM followed by the dequantisation epilogue."""
    return dequantize(int8_matmul(xq, wq), x_scale, w_scale, out)


def smoothquant_linear(x, s, wq, w_scale, out: str = "bf16"):
    """The run-time path: quantise X per token (with 1/s), int8 GEMM, dequantise.

    Returns (y, xq, x_scale, acc).
    """
    xq, dx = quantize_activations(x, s)
    acc = int8_matmul(xq, wq)
    return dequantize(acc, dx, w_scale, out), xq, dx, acc


# --------------------------------------------------------------------------
# Baselines used only to order quantisation errors
# --------------------------------------------------------------------------
def per_tensor_int8_linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Naive W8A8: one scale for all of X and one for all of W, no smoothing.

    The W8A8 post, "Why Activation Quantization Is Hard ..." and the LLM.int8()
    page, "Why architecture matters here": a single scale sized for the
    outlier. Returned in binary64 (an error baseline, not a kernel result).
    """
    x = _f32(x)
    w = _f32(w)
    sx = F32(np.abs(x).max() / F32(QMAX))
    sw = F32(np.abs(w).max() / F32(QMAX))
    xq = np.clip(np.rint((x / sx).astype(F32)), -QMAX, QMAX)
    wq = np.clip(np.rint((w / sw).astype(F32)), -QMAX, QMAX)
    return (xq.astype(np.float64) @ wq.astype(np.float64)) * float(sx) * float(sw)
