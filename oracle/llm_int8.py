"""CPU oracle of the LLM.int8() vectorwise decomposition (test infrastructure only).

Follows the LLM.int8() page, sections "The architecture: every piece
explained" and "End-to-end flow", in its order:

1. detection: a feature column is an outlier when any |x| in it is strictly
   greater than the threshold (6.0 is the canonical value);
2. column split: outlier columns go to the fp16 path, the rest to int8;
3. int8 path: one scale per row of X over the regular columns only, one scale
   per column of W (made once at load time over all of W's rows); int8 x int8
   with an int32 accumulator; dequantisation by the row scale times the
   column scale, to fp16;
4. fp16 path: the outlier columns of X times the matching fp16 weight rows;
5. accumulate: the two fp16 partial products are added.

Readings (listed with reasons in the design notes):

* The int8 path keeps all K columns and sets the outlier columns of Xq to 0;
  that is the same sum as dropping them (the split is linear).
* The fp16 slice takes fp16 inputs, multiplies and adds in binary32 in
  ascending outlier-column order (one rounding per multiply and per add), and
  rounds the sum to fp16.
* The final sum is the exact sum of the two fp16 partials, rounded once to
  fp16.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .smoothquant import QMAX, F32, int8_matmul


def detect_outliers(x: np.ndarray, threshold: float) -> np.ndarray:
    """Boolean mask over feature columns: max_i |x_ic| > threshold (strict)."""
    x = np.asarray(x, dtype=np.float32)
    colmax = np.abs(x).max(axis=0) if x.shape[0] else np.zeros(x.shape[1], F32)
    return colmax > F32(threshold)


def quantize_rows_regular(x: np.ndarray, mask: np.ndarray):
    """Row-wise int8 over the regular columns; outlier columns of Xq are 0."""
    xr = np.where(mask[None, :], F32(0), np.asarray(x, dtype=np.float32)).astype(F32)
    rowmax = np.abs(xr).max(axis=1).astype(F32) if xr.shape[1] else np.zeros(xr.shape[0], F32)
    scale = (rowmax / F32(QMAX)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (xr / scale[:, None]).astype(F32)
    q = np.clip(np.rint(ratio), -QMAX, QMAX)
    q = np.where((scale[:, None] > 0) & ~mask[None, :], q, 0.0)
    return q.astype(np.int8), scale


def fp16_outlier_product(x: np.ndarray, w16: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """fp16(sum over outlier columns c, ascending, of x_ic * w_cn), binary32 accumulation."""
    x = np.asarray(x, dtype=np.float32)
    w = np.asarray(w16, dtype=np.float32)
    acc = np.zeros((x.shape[0], w.shape[1]), dtype=F32)
    for c in np.flatnonzero(mask):
        prod = (x[:, c:c + 1] * w[c:c + 1, :]).astype(F32)
        acc = (acc + prod).astype(F32)
    return acc.astype(np.float16)


def int8_decomp_linear(x: np.ndarray, wq: np.ndarray, w_scale: np.ndarray,
                       w16: np.ndarray, threshold: float = 6.0,
                       mask: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The decomposed linear layer. Returns every intermediate by name.

    x: [M x K] fp16 values; wq: [N x K] int8 (per-column scales over all K
    rows, made at load time); w_scale: [N]; w16: [K x N] fp16 weights.
    ``mask`` replaces the detection step when the outlier columns are already
    known (for example from all rows of a matrix whose rows are evaluated one
    subset at a time; every later step is row-independent).
    """
    if mask is None:
        mask = detect_outliers(x, threshold)
    xq, dx = quantize_rows_regular(x, mask)
    acc = int8_matmul(xq, wq)
    y = (acc.astype(F32) * dx[:, None]).astype(F32)
    y = (y * np.asarray(w_scale, dtype=F32)[None, :]).astype(F32)
    y_int = y.astype(np.float16)
    y_out = fp16_outlier_product(x, w16, mask)
    y_sum = (y_int.astype(np.float64) + y_out.astype(np.float64)).astype(np.float16)
    return dict(y=y_sum, mask=mask, count=int(mask.sum()), xq=xq, x_scale=dx, acc=acc,
                y_int=y_int, y_out=y_out)
