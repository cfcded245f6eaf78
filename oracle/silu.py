"""CPU oracle of the gated-MLP activation feeding the down projection, fused
with its smoothing divide and per-token int8 quantisation (test
infrastructure only).

The pages quantise every linear layer's input per token at run time ("Half
the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8 LLM
Quantization", sections "How the Model Was Compressed" and "Why Activation
Quantization Is Hard"), with the smoothing divide of "How the smoothing factor
is computed", and blame the memory-bound quantisation steps for the
inter-token latency cost ("Performance After Quantization", Inter-Token
Latency). For the down projection of a gated MLP that input is
h = SiLU(gate) * up, made from the gate and up projections' outputs. The
pages name neither SiLU nor its arithmetic, so every detail below is a
reading (listed in the design notes):

* gate and up are the bf16 outputs of the gate/up projection (the storage
  type of the model's activations); h is formed in binary32 and rounded to
  bf16, the type it would be stored in between two kernels; the quantiser
  then sees exactly what an unfused pipeline would hand it.
* SiLU(z) = z * sigma(z), sigma(z) = 1 / (1 + e^-z), every step one IEEE
  binary32 operation: e^t is evaluated by a fixed algorithm (below) so that
  any implementation following the same steps reproduces it bit for bit.
  Argument reduction (Cody and Waite): t = k ln2 + r with k = rint(t * RN32(1/ln2))
  (round half to even), r = (t - k L1) - k L2, where ln2 = L1 + L2 and L1
  has 16 significant bits, so k L1 is exact for every |k| < 2^8 that occurs;
  e^r by the degree-7 Taylor polynomial in Horner form with the binary32
  coefficients RN32(1/n!); e^t = p(r) * 2^k (ldexp: exact scaling, correctly
  rounded into the subnormal range). t > 100 gives +inf and t < -110 gives 0
  (beyond binary32's range either way). Over the normal range this e^t is
  within 1.2 binary32 ulp of the true value.
* No fused multiply-add anywhere (each product and sum rounds on its own).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .numerics import round_bf16
from .smoothquant import quantize_activations

F32 = np.float32

# ln2 = L1 + L2: L1 holds 16 significant bits, so k * L1 is exact for |k| < 2^8
# (|t| <= 110 gives |k| <= 159).
LN2_HI = F32(0.693145751953125)           # 0x3F317200
LN2_LO = F32(1.428606765330187e-06)       # ln2 - LN2_HI rounded to binary32
INV_LN2 = F32(1.4426950408889634)         # RN32(1/ln2)
# 1/n! for n = 7 .. 0, rounded to binary32 (Horner from the highest degree)
EXP_COEF = [F32(1.0 / 5040.0), F32(1.0 / 720.0), F32(1.0 / 120.0), F32(1.0 / 24.0), F32(1.0 / 6.0),
            F32(0.5), F32(1.0), F32(1.0)]
T_HI = F32(100.0)
T_LO = F32(-110.0)


def exp32(t: np.ndarray) -> np.ndarray:
    """e^t in binary32 by the fixed algorithm of the module notes."""
    t = np.asarray(t, dtype=F32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):  # out-of-range t: replaced below
        k = np.rint((t * INV_LN2).astype(F32)).astype(F32)
        k = np.clip(k, F32(-256), F32(256))
        r = ((t - (k * LN2_HI).astype(F32)).astype(F32) - (k * LN2_LO).astype(F32)).astype(F32)
        p = np.full_like(r, EXP_COEF[0])
        for c in EXP_COEF[1:]:
            p = ((p * r).astype(F32) + c).astype(F32)
        e = np.ldexp(p, k.astype(np.int32)).astype(F32)
    e = np.where(t > T_HI, F32(np.inf), e)
    e = np.where(t < T_LO, F32(0.0), e)
    return e.astype(F32)


def silu32(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * (1 / (1 + e^-z)), one binary32 operation per step."""
    z = np.asarray(z, dtype=F32)
    e = exp32(-z)
    with np.errstate(over="ignore", divide="ignore"):
        sig = (F32(1.0) / (F32(1.0) + e).astype(F32)).astype(F32)
    return (z * sig).astype(F32)


def gated_activation(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """h = RN_bf16(RN32(SiLU(gate) * up)), returned as binary32 holding bf16 values."""
    g = np.asarray(gate, dtype=F32)
    u = np.asarray(up, dtype=F32)
    return round_bf16((silu32(g) * u).astype(F32))


def silu_mul_quantize(gate: np.ndarray, up: np.ndarray, s: Optional[np.ndarray] = None
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """The down projection's input h, smoothed and quantised per token:
    quantize_activations(gated_activation(gate, up), s)."""
    return quantize_activations(gated_activation(gate, up), s)
