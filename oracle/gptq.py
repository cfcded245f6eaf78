"""CPU oracle of GPTQ weight rounding (test infrastructure only).

"Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8 LLM
Quantization":
* "How the Model Was Compressed": GPTQ runs after SmoothQuant and sets the
  int8 weight values, using error compensation.
* "How the smoothing factor is computed": the weights it starts from are the
  smoothed ones (row j times s_j).
* "How GPTQ improves on naive quantization" gives the per-layer steps:
  1. a Hessian from the calibration activations;
  2. quantise one weight and measure its rounding error;
  3. spread that error over the weights not yet quantised, weighted by the
     Hessian (less onto the sensitive ones);
  4. repeat until every weight is quantised.
  It cites Frantar et al., "GPTQ" (2022), for the algorithm. This module
  follows that paper's procedure.

The pages leave the numerical details open. The readings below are listed in
the design notes:

* H = sum over calibration rows t of x_t x_t^T (K x K), where x_t are the
  smoothed activations fl32(x / s) the layer sees. It is computed in binary64:
  products of binary32 values are exact there. The paper's factor 2/T is
  left out; the result does not depend on a positive factor of H.
* Inputs j with H_jj = 0 are dead (no calibration signal): their weights are
  set to 0 and H_jj to 1.
* Damping lambda = 0.01 * mean(diag H) is added to the diagonal. This is the
  paper's default; it keeps H^-1 well defined.
* The weights are processed in input order j = 0 .. K-1 (no reordering). Each
  output channel n (weight column) is independent and keeps the RTN scale
  fixed before the sweep: sw_n = fl32(max_j |W'_jn| / 127), over the weights
  after the dead-input zeroing.
* With U the upper Cholesky factor of H^-1 (H^-1 = U^T U), step j does, for
  every n:
    q_jn = clamp(round_half_even(w_jn / sw_n), -127, 127), or 0 when sw_n = 0
    e_jn = (w_jn - q_jn * sw_n) / U_jj
    w_in -= e_jn * U_ji            for every i > j
  where w is the running (compensated) weight. All of this is in binary64;
  the paper's own code uses binary32.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .smoothquant import QMAX, smooth_activations

F32 = np.float32
GPTQ_DAMP = 0.01


def gptq_hessian(x_cal: np.ndarray, s: Optional[np.ndarray] = None) -> np.ndarray:
    """H = X^T X over the smoothed calibration activations X = fl32(x / s), in binary64."""
    xh = smooth_activations(x_cal, s).astype(np.float64)
    return xh.T @ xh


def gptq_quantize(w_folded: np.ndarray, h: np.ndarray, damp: float = GPTQ_DAMP, trace: bool = False):
    """GPTQ of the smoothed weights W' [K x N] (binary32) against the Hessian H [K x K].

    Returns (Wq [N x K] int8, the transpose like the RTN weights; sw [N] binary32).
    With trace=True, it also returns z [K x N]: the compensated weight that
    step j rounds, in binary64.
    """
    w = np.asarray(w_folded, dtype=F32).astype(np.float64)
    k, n = w.shape
    h = np.array(h, dtype=np.float64, copy=True)
    dead = np.diag(h) == 0
    h[dead, dead] = 1.0
    w[dead, :] = 0.0
    colmax = np.abs(w.astype(F32)).max(axis=0).astype(F32) if k else np.zeros(n, F32)
    sw = (colmax / F32(QMAX)).astype(F32)
    sw64 = sw.astype(np.float64)
    h[np.diag_indices(k)] += damp * np.mean(np.diag(h))
    hinv = np.linalg.inv(h)
    u = np.linalg.cholesky(hinv).T                       # upper, H^-1 = U^T U
    codes = np.zeros((k, n), dtype=np.int8)
    z = np.zeros((k, n), dtype=np.float64)
    for j in range(k):
        wj = w[j, :].copy()
        z[j] = wj
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(sw64 > 0, np.clip(np.rint(wj / sw64), -QMAX, QMAX), 0.0)
        codes[j] = q.astype(np.int8)
        err = (wj - q * sw64) / u[j, j]
        w[j + 1:, :] -= np.outer(u[j, j + 1:], err)
    out = (np.ascontiguousarray(codes.T), sw)
    return out + (z,) if trace else out


def gptq_smooth_quantize(x_cal: np.ndarray, s: Optional[np.ndarray], w: np.ndarray,
                         damp: float = GPTQ_DAMP) -> Tuple[np.ndarray, np.ndarray]:
    """The whole offline step for one layer: W' = fl32(s_j * W_jn) (W itself
    without s), H from fl32(x / s), then the GPTQ sweep."""
    w = np.asarray(w, dtype=F32)
    wf = w.copy() if s is None else (np.asarray(s, F32)[:, None] * w).astype(F32)
    return gptq_quantize(wf, gptq_hessian(x_cal, s), damp)
