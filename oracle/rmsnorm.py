"""CPU oracle of the RMSNorm whose gain carries the smoothing factor, followed
by per-token int8 quantisation (test infrastructure only).

The pages cited, from "Half the Size, Better Performance, Same Accuracy:
Understanding W8A8 INT8 LLM Quantization" (the W8A8 post):

* "Where the outlier actually comes from": RMSNorm first divides every value
  of a token's vector by that vector's root-mean-square, then multiplies
  channel j by a learned per-channel gain gamma_j, the same for every token.
  Its worked example multiplies the normalised values by gamma elementwise.
* "How the smoothing factor is computed", last paragraph: SmoothQuant divides
  gamma by s and multiplies the matching weight row by s, so the activation
  leaves the norm already divided by s and no run-time division is needed.
* "How the Model Was Compressed" / "Why Activation Quantization Is Hard": the
  per-token quantisation that follows (quantize_activations of smoothquant.py).

Readings taken where the pages fix no detail (each is listed in the design
notes with its reason):

* rms = sqrt(mean_j x_j^2 + eps), with eps >= 0 a binary32 parameter. eps = 0
  is the pages' definition as written; models add a small eps, so it is an
  argument.
* The sum of squares is exact: each square of a binary32 (hence bf16 or fp16)
  value is exact in binary64, and math.fsum returns their exact sum rounded
  once to binary64. The rest of the scalar chain is binary64, one IEEE
  operation at a time: mean = S / K, v = mean + eps, r = sqrt(v),
  inv = 1 / r; then inv32 = RN32(inv).
* The normalised value is RN32(x_j * inv32) and the activation
  RN32(normalised_j * g_j) with g = the folded gain, both in binary32.
* A row with v == 0 (all zero and eps == 0), or whose inv32 overflows binary32
  (v below 2^-256, only reachable with eps == 0), normalises to zero.
* The folded gain is g_j = RN32(gamma_j / s_j) (gamma_j itself without s).
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .smoothquant import quantize_activations

F32 = np.float32


def _f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32)


def fold_norm_gain(gamma: np.ndarray, s: Optional[np.ndarray]) -> np.ndarray:
    """g_j = fl32(gamma_j / s_j): the smoothing factor moved into the norm's gain.

    The W8A8 post, "How the smoothing factor is computed" (gamma is divided by
    s) and the smoothed example of "Where the outlier actually comes from".
    """
    g = _f32(gamma)
    if s is None:
        return g.copy()
    return (g / _f32(s)).astype(F32)


def rms_inverse(x: np.ndarray, eps: float = 0.0) -> np.ndarray:
    """inv32_i = RN32(1 / sqrt(mean_j x_ij^2 + eps)) per row, by the chain above.

    The W8A8 post, "Where the outlier actually comes from" (every value is
    divided by the vector's root-mean-square). Returns binary32 [M]; a
    degenerate row (see the module notes) gets 0.
    """
    x = _f32(x)
    m, k = x.shape
    e = float(F32(eps))
    out = np.zeros(m, F32)
    for i in range(m):
        sq = np.square(x[i].astype(np.float64))  # exact: 48-bit significands, exponents in range
        s = math.fsum(sq.tolist())
        v = s / k + e
        if not v > 0.0:
            continue
        inv = 1.0 / math.sqrt(v)
        with np.errstate(over="ignore"):
            inv32 = F32(inv)
        if np.isfinite(inv32):
            out[i] = inv32
    return out


def apply_gain(normalized: np.ndarray, gain: np.ndarray) -> np.ndarray:
    """a_ij = fl32(n_ij * g_j): the channel-wise gain of RMSNorm.

    The W8A8 post, "Where the outlier actually comes from" (activation =
    normalized x gamma, elementwise).
    """
    return (_f32(normalized) * _f32(gain)[None, :]).astype(F32)


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float = 0.0) -> np.ndarray:
    """RMSNorm in binary32: a_ij = fl32(fl32(x_ij * inv32_i) * g_j)."""
    x = _f32(x)
    inv = rms_inverse(x, eps)
    n = (x * inv[:, None]).astype(F32)
    return apply_gain(n, gain)


def rmsnorm_quantize(x: np.ndarray, gain: np.ndarray, eps: float = 0.0) -> Tuple[np.ndarray, np.ndarray]:
    """RMSNorm with the folded gain, then per-token int8 quantisation.

    The activation a = rmsnorm(x, g) is already divided by s through g, so it
    is quantised as it stands: d_i = fl32(max_j |a_ij| / 127),
    q_ij = clamp(round_half_even(fl32(a_ij / d_i)), -127, 127).
    Returns (Xq [M x K] int8, x_scale [M] binary32).
    """
    return quantize_activations(rmsnorm(x, gain, eps))
