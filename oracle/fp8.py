"""CPU oracle of the FP8 (E4M3) W8A8 variant (test infrastructure only).

"Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
LLM Quantization", section "Conclusion" ("When W8A8 INT8 is a good fit" and
"What to explore next"): FP8 quantisation is the alternative that skips the
calibration algorithms (SmoothQuant, GPTQ) and needs newer hardware. The
pages give no format or scaling details; the readings below are listed in the
design notes:

* Format: E4M3 with the OCP "fn" encoding (1 sign, 4 exponent bits with bias
  7, 3 mantissa bits; no infinities; the largest finite magnitude is 448;
  subnormals m * 2^-9). The matrix cores this targets take it natively.
* Scales as in the int8 path with 448 in place of 127: one scale per token
  over all channels, d_i = fl32(max_j |x_ij| / 448), and one per output
  channel for the weights, sw_n = fl32(max_k |W_kn| / 448). No smoothing.
* Codes: v = fl32(x / d), then the E4M3 value nearest to v, ties to the even
  mantissa; |v| <= 448 (up to the rounding of the quotient) by construction.
  A zero scale gives zero codes.
* Product: acc = sum_k xq_ik * wq_nk over the E4M3 values. Every product of
  two E4M3 values is exact in binary32; the sum is taken exactly here
  (binary64 suffices: 4-bit significands, exponents within 2^-18 .. 2^18).
  The matrix cores sum in binary32, so the GPU's acc differs from this one
  by rounding only, which the parity tests bound.
* Dequantisation as in the int8 path: y = out(fl32(fl32(acc * d_i) * sw_n)).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .numerics import round_to

F32 = np.float32
E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The binary64 value of each of the 256 E4M3 codes (NaN for 0x7F / 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** -9
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each binary32 v (ties to the even mantissa), with
    magnitudes above 448 taken to 448 (they do not occur in the quantisers:
    |v| <= 448 up to one rounding)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    # exponent of the binade, normals from 2^-6; below that the subnormal spacing 2^-9
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    e = np.clip(e, -6, 8)
    step = np.exp2(e - 3.0)                       # spacing of the binade (subnormals: 2^-9)
    q = a / step                                  # exact: a power-of-two division
    n = np.floor(q)
    frac = q - n
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(n, 2) == 1))
    n = n + up
    r = n * step                                  # the rounded magnitude, exact
    # carry into the next binade is a valid value (it is representable)
    ef = np.floor(np.log2(np.where(r > 0, r, 1.0))).astype(np.int64)
    ef = np.where(r >= 2.0 ** -6, ef, -7)         # -7 marks a subnormal (field 0)
    man = np.where(ef >= -6, np.rint(r / np.exp2(ef) * 8.0) - 8.0, np.rint(r / 2.0 ** -9))
    field = np.where(ef >= -6, ef + 7, 0)
    code = sign | (field << 3) | man.astype(np.int64)
    code = np.where(r == 0, sign, code)
    return code.astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """binary32 value of each E4M3 code (exact)."""
    return e4m3_values()[np.asarray(code, dtype=np.uint8)].astype(F32)


def quantize_activations_fp8(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token E4M3: d_i = fl32(max_j |x_ij| / 448), q_ij = E4M3(fl32(x_ij / d_i)).
    Returns (codes [M x K] uint8, d [M] binary32)."""
    x = np.asarray(x, dtype=F32)
    rowmax = np.abs(x).max(axis=1).astype(F32) if x.shape[1] else np.zeros(x.shape[0], F32)
    d = (rowmax / F32(E4M3_MAX)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (x / d[:, None]).astype(F32)
    codes = e4m3_encode(np.where(d[:, None] > 0, v, F32(0)))
    return codes, d


def quantize_weights_fp8(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-output-channel E4M3 of W [K x N]: sw_n = fl32(max_k |W_kn| / 448),
    codes stored transposed [N x K] like the int8 weights."""
    w = np.asarray(w, dtype=F32)
    colmax = np.abs(w).max(axis=0).astype(F32)
    sw = (colmax / F32(E4M3_MAX)).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (w / sw[None, :]).astype(F32)
    codes = e4m3_encode(np.where(sw[None, :] > 0, v, F32(0)))
    return np.ascontiguousarray(codes.T), sw


def fp8_matmul(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc_in = sum_k E4M3(xq_ik) * E4M3(wq_nk), exact (binary64)."""
    a = e4m3_decode(xq).astype(np.float64)
    b = e4m3_decode(wq).astype(np.float64)
    return a @ b.T


def fp8_linear(xq, x_scale, wq, w_scale, out: str = "bf16") -> np.ndarray:
    """y = out(fl32(fl32(fl32(acc) * d_i) * sw_n)) with the exact acc rounded once to binary32."""
    acc = fp8_matmul(xq, wq).astype(F32)
    y = (acc * np.asarray(x_scale, F32)[:, None]).astype(F32)
    y = (y * np.asarray(w_scale, F32)[None, :]).astype(F32)
    return round_to(y, out)
