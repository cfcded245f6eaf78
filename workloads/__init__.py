"""Seeded synthetic inputs for the W8A8 linear layer and the LLM.int8() variant.

This module only draws random numbers and shapes them; it computes none of the
quantisation method. Both the CPU oracle (through the tests) and the HIP path
receive exactly the arrays produced here.

Every tensor comes from its own child of ``numpy.random.SeedSequence(seed)``,
so changing one shape never changes another tensor's values.

Activation models (stand-ins for the pages' Llama-3.1-8B activations, which are
not available):

* ``gaussian_outlier``: X ~ N(0, 1) with a few persistent channels multiplied
  by a large factor. Persistent per-channel outliers that come from the norm
  gain are the structure described in "Half the Size, Better Performance, Same
  Accuracy: Understanding W8A8 INT8 LLM Quantization", section "Where the
  outlier actually comes from"; about one feature in a thousand with magnitude
  near 60 is the picture in the LLM.int8() page, section "Why architecture
  matters here".
* ``silu_gated``: h = SiLU(a) * b with a, b ~ N(0, 1) independent (the input
  of a gated MLP's down projection), heavy tailed, with the outlier channels
  multiplied by 40.
* ``correlated_outlier``: X = Z + L M with Z ~ N(0, 1), 32 latent factors
  L ~ N(0, 1) per row and a fixed mixing M ~ N(0, 0.25) per layer, then the
  outlier channels multiplied by 60. The channels are correlated, as a real
  layer's inputs are, so GPTQ's Hessian (its calibration input for "How
  GPTQ improves on naive quantization") is far from diagonal; with
  uncorrelated channels GPTQ would pass almost no error on.
* ``llm_int8``: X ~ N(0, 1) fp16 with 8 columns multiplied by magnitudes
  spread evenly over [6, 60], so every one of them crosses the 6.0 threshold.
* RMSNorm inputs (``norm_case``): the residual stream before the norm, rows
  x ~ N(0, 1) times a per-row magnitude exp(N(0, 1)) (tokens of different
  RMS); the gain gamma ~ U(0.5, 1.5) with the outlier channels set to values
  in [20, 100]. "Where the outlier actually comes from" shows exactly this: a
  balanced normalised vector and one gain of 100 that makes the outlier.
  ``wide_range_rows`` gives rows whose binary exponents spread over a chosen
  range, with zeros, for exercising the exact sum of squares.
* Gate/up projection outputs (``gate_up_case``): gate ~ N(0, 2^2), up ~ N(0, 1)
  in bf16, with about 1% of the gate values replaced by magnitudes in
  [15, 120] of either sign (SiLU's saturated regions and the exponential's
  overflow and underflow), and the persistent outlier channels of the up side
  scaled by 20.

Weights are N(0, 0.02) in every configuration.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "LinearCase",
    "Int8DecompCase",
    "outlier_channels",
    "activations",
    "weights",
    "linear_case",
    "decomp_case",
    "random_linear_case",
    "NormCase",
    "norm_case",
    "wide_range_rows",
    "GateUpCase",
    "gate_up_case",
    "GptqCase",
    "gptq_case",
    "CONFIGS",
]

# Streams drawn from each seed, by role.
_STREAM = {"calib": 0, "x": 1, "w": 2, "outliers": 3, "extra": 4}


def _rng(seed: int, role, stream: int = 0) -> np.random.Generator:
    """Generator for one tensor: role names the tensor, ``stream`` separates extra draws."""
    idx = _STREAM[role] + stream
    child = np.random.SeedSequence(seed).spawn(idx + 1)[idx]
    return np.random.default_rng(child)


def _as_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp32 array to ``dtype`` and return it as exactly representable fp32.

    The rounding is the input format's own conversion (torch's CPU cast), used
    only to produce inputs of the stated storage type.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return torch.from_numpy(a).to(tdt).to(torch.float32).numpy()


def outlier_channels(k: int, seed: int = 0, fixed: Optional[Sequence[int]] = None) -> np.ndarray:
    """Indices of the persistent outlier channels: about 0.1% of ``k``, at least one."""
    if fixed is not None:
        return np.asarray(sorted(fixed), dtype=np.int64)
    n = max(1, int(round(0.001 * k)))
    return np.sort(_rng(seed, "outliers").choice(k, n, replace=False)).astype(np.int64)


def activations(rows: int, k: int, model: str, seed: int, role: str,
                channels: np.ndarray, dtype: str) -> np.ndarray:
    """Activation rows [rows x k] for one of the activation models above."""
    g = _rng(seed, role)
    if model == "gaussian_outlier":
        x = g.standard_normal((rows, k), dtype=np.float32)
        x[:, channels] *= np.float32(60.0)
    elif model == "silu_gated":
        a = g.standard_normal((rows, k), dtype=np.float32)
        b = g.standard_normal((rows, k), dtype=np.float32)
        x = (a / (1.0 + np.exp(-a.astype(np.float64)))).astype(np.float32) * b
        x[:, channels] *= np.float32(40.0)
    elif model == "correlated_outlier":
        # channels share 32 latent directions (the same mixing for every row
        # of a layer), so the calibration Hessian is far from diagonal
        z = g.standard_normal((rows, k), dtype=np.float32)
        lat = g.standard_normal((rows, 32), dtype=np.float32)
        mix = _rng(seed, "extra", 300).standard_normal((32, k), dtype=np.float32) * np.float32(0.5)
        x = z + lat @ mix
        x[:, channels] *= np.float32(60.0)
    elif model == "llm_int8":
        x = g.standard_normal((rows, k), dtype=np.float32)
        mags = np.linspace(6.0, 60.0, len(channels)).astype(np.float32)
        x[:, channels] *= mags[None, :]
    else:
        raise ValueError(f"unknown activation model {model!r}")
    return _as_dtype(x, dtype)


def weights(k: int, n: int, seed: int, dtype: str, std: float = 0.02) -> np.ndarray:
    """W [k x n] ~ N(0, std), rows are input channels, columns output channels."""
    g = _rng(seed, "w")
    w = g.standard_normal((k, n), dtype=np.float32) * np.float32(std)
    return _as_dtype(w, dtype)


@dataclasses.dataclass
class LinearCase:
    """One smoothed W8A8 linear workload: calibration rows, measured rows, weight."""

    name: str
    m: int
    k: int
    n: int
    x_dtype: str
    w_dtype: str
    y_dtype: str
    alpha: float
    channels: np.ndarray
    x_calib: np.ndarray  # [t x k] fp32 holding x_dtype values
    x: np.ndarray        # [m x k]
    w: np.ndarray        # [k x n]
    model: str
    seed: int


@dataclasses.dataclass
class Int8DecompCase:
    name: str
    m: int
    k: int
    n: int
    threshold: float
    channels: np.ndarray
    x: np.ndarray  # [m x k] fp32 holding fp16 values
    w: np.ndarray  # [k x n] fp32 holding fp16 values
    seed: int


# The five workloads.  Entries give (m, k, n, dtypes, activation model,
# calibration rows, alpha list).
CONFIGS: Dict[str, dict] = {
    "tiny": dict(m=16, k=256, n=512, x_dtype="f32", w_dtype="f32", y_dtype="f32",
                 model="gaussian_outlier", calib_rows=64, alphas=[0.5], fixed=(7, 131)),
    "qkv_prefill": dict(m=2048, k=4096, n=6144, x_dtype="bf16", w_dtype="bf16", y_dtype="bf16",
                        model="gaussian_outlier", calib_rows=8 * 512, alphas=[0.5]),
    "gateup_prefill": dict(m=8192, k=4096, n=28672, x_dtype="bf16", w_dtype="bf16", y_dtype="bf16",
                           model="gaussian_outlier", calib_rows=8 * 512, alphas=[0.5, 0.8]),
    "down_prefill": dict(m=8192, k=14336, n=4096, x_dtype="bf16", w_dtype="bf16", y_dtype="bf16",
                         model="silu_gated", calib_rows=8 * 512, alphas=[0.5, 0.8]),
    "decode_up": dict(m=64, k=4096, n=14336, x_dtype="bf16", w_dtype="bf16", y_dtype="bf16",
                      model="gaussian_outlier", calib_rows=8 * 512, alphas=[0.5], ms=[1, 8, 32, 64]),
    "decode_down": dict(m=64, k=14336, n=4096, x_dtype="bf16", w_dtype="bf16", y_dtype="bf16",
                        model="silu_gated", calib_rows=8 * 512, alphas=[0.5], ms=[1, 8, 32, 64]),
    "llm_int8": dict(m=4096, k=8192, n=8192, threshold=6.0, n_outlier_cols=8),
}


def linear_case(name: str, seed: int = 0, m: Optional[int] = None, alpha: Optional[float] = None,
                calib_rows: Optional[int] = None) -> LinearCase:
    cfg = CONFIGS[name]
    m = cfg["m"] if m is None else m
    k, n = cfg["k"], cfg["n"]
    ch = outlier_channels(k, seed, cfg.get("fixed"))
    t = cfg["calib_rows"] if calib_rows is None else calib_rows
    xc = activations(t, k, cfg["model"], seed, "calib", ch, cfg["x_dtype"])
    x = activations(m, k, cfg["model"], seed, "x", ch, cfg["x_dtype"])
    w = weights(k, n, seed, cfg["w_dtype"])
    return LinearCase(name=name, m=m, k=k, n=n, x_dtype=cfg["x_dtype"], w_dtype=cfg["w_dtype"],
                      y_dtype=cfg["y_dtype"], alpha=cfg["alphas"][0] if alpha is None else alpha,
                      channels=ch, x_calib=xc, x=x, w=w, model=cfg["model"], seed=seed)


def random_linear_case(m: int, k: int, n: int, seed: int, dtype: str = "bf16",
                       model: str = "gaussian_outlier", calib_rows: int = 256,
                       alpha: float = 0.5, y_dtype: Optional[str] = None) -> LinearCase:
    """A smaller workload with the same recipe, for ragged and multi-tile shapes."""
    ch = outlier_channels(k, seed)
    xc = activations(calib_rows, k, model, seed, "calib", ch, dtype)
    x = activations(m, k, model, seed, "x", ch, dtype)
    w = weights(k, n, seed, dtype)
    return LinearCase(name=f"rand_{m}x{k}x{n}_s{seed}", m=m, k=k, n=n, x_dtype=dtype, w_dtype=dtype,
                      y_dtype=y_dtype or dtype, alpha=alpha, channels=ch, x_calib=xc, x=x, w=w,
                      model=model, seed=seed)


@dataclasses.dataclass
class GptqCase:
    """Calibration rows and the weight of one layer for GPTQ."""
    k: int
    n: int
    t: int
    dtype: str
    channels: np.ndarray
    dead: Tuple[int, ...]  # inputs whose calibration column is zero
    x_calib: np.ndarray  # [t x k] fp32 holding dtype values
    w: np.ndarray  # [k x n]


def gptq_case(k: int, n: int, t: int, seed: int, dtype: str = "bf16", dead: Sequence[int] = (),
              model: str = "correlated_outlier") -> GptqCase:
    ch = outlier_channels(k, seed)
    xc = activations(t, k, model, seed, "calib", ch, dtype)
    for j in dead:
        xc[:, j] = 0.0
    return GptqCase(k=k, n=n, t=t, dtype=dtype, channels=ch, dead=tuple(dead), x_calib=xc,
                    w=weights(k, n, seed, dtype))


@dataclasses.dataclass
class NormCase:
    """RMSNorm input rows, the norm's gain and calibration rows."""

    m: int
    k: int
    dtype: str
    channels: np.ndarray
    x: np.ndarray        # [m x k] fp32 holding dtype values (the residual stream)
    gamma: np.ndarray    # [k] fp32 holding dtype values
    x_calib: np.ndarray  # [t x k]


def _residual_rows(g: np.random.Generator, rows: int, k: int) -> np.ndarray:
    x = g.standard_normal((rows, k), dtype=np.float32)
    return x * np.exp(g.standard_normal((rows, 1))).astype(np.float32)


def norm_case(m: int, k: int, seed: int, dtype: str = "bf16", calib_rows: int = 256) -> NormCase:
    ch = outlier_channels(k, seed)
    gg = _rng(seed, "extra", 300)
    gamma = gg.uniform(0.5, 1.5, size=k).astype(np.float32)
    gamma[ch] = gg.uniform(20.0, 100.0, size=len(ch)).astype(np.float32)
    x = _residual_rows(_rng(seed, "x"), m, k)
    xc = _residual_rows(_rng(seed, "calib"), calib_rows, k)
    return NormCase(m=m, k=k, dtype=dtype, channels=ch, x=_as_dtype(x, dtype), gamma=_as_dtype(gamma, dtype),
                    x_calib=_as_dtype(xc, dtype))


def wide_range_rows(m: int, k: int, seed: int, dtype: str, lo_exp: int, hi_exp: int,
                    zero_frac: float = 0.1) -> np.ndarray:
    """Rows [m x k] of values m * 2^e, e uniform in [lo_exp, hi_exp] (clipped to
    what ``dtype`` represents), random signs and significands, some zeros."""
    g = _rng(seed, "extra", 400)
    mant = g.uniform(1.0, 2.0, size=(m, k))
    e = g.integers(lo_exp, hi_exp + 1, size=(m, k))
    x = mant * np.exp2(e.astype(np.float64)) * g.choice([-1.0, 1.0], size=(m, k))
    x[g.random((m, k)) < zero_frac] = 0.0
    lim = {"bf16": 3.0e38, "f32": 3.0e38, "f16": 60000.0}[dtype]
    x = np.clip(x, -lim, lim).astype(np.float32)
    return _as_dtype(x, dtype)


@dataclasses.dataclass
class GateUpCase:
    """bf16 outputs of a gate/up projection (the down projection's input side)."""

    m: int
    k: int
    channels: np.ndarray
    gate: np.ndarray        # [m x k] fp32 holding bf16 values
    up: np.ndarray          # [m x k]
    gate_calib: np.ndarray  # [t x k]
    up_calib: np.ndarray


def _gate_up_rows(g: np.random.Generator, rows: int, k: int, ch: np.ndarray):
    gate = g.standard_normal((rows, k), dtype=np.float32) * np.float32(2.0)
    wild = g.random((rows, k)) < 0.01
    mags = g.uniform(15.0, 120.0, size=(rows, k)).astype(np.float32) * g.choice([-1.0, 1.0], size=(rows, k))
    gate = np.where(wild, mags.astype(np.float32), gate)
    up = g.standard_normal((rows, k), dtype=np.float32)
    up[:, ch] *= np.float32(20.0)
    return _as_dtype(gate, "bf16"), _as_dtype(up, "bf16")


def gate_up_case(m: int, k: int, seed: int, calib_rows: int = 256) -> GateUpCase:
    ch = outlier_channels(k, seed)
    gate, up = _gate_up_rows(_rng(seed, "x"), m, k, ch)
    gc, uc = _gate_up_rows(_rng(seed, "calib"), calib_rows, k, ch)
    return GateUpCase(m=m, k=k, channels=ch, gate=gate, up=up, gate_calib=gc, up_calib=uc)


def decomp_case(seed: int = 0, m: Optional[int] = None, k: Optional[int] = None,
                n: Optional[int] = None, n_outlier_cols: Optional[int] = None) -> Int8DecompCase:
    cfg = CONFIGS["llm_int8"]
    m = cfg["m"] if m is None else m
    k = cfg["k"] if k is None else k
    n = cfg["n"] if n is None else n
    nc = cfg["n_outlier_cols"] if n_outlier_cols is None else n_outlier_cols
    ch = np.sort(_rng(seed, "outliers").choice(k, nc, replace=False)).astype(np.int64) if nc else \
        np.zeros(0, dtype=np.int64)
    x = activations(m, k, "llm_int8", seed, "x", ch, "f16")
    w = weights(k, n, seed, "f16")
    return Int8DecompCase(name=f"llm_int8_{m}x{k}x{n}", m=m, k=k, n=n, threshold=cfg["threshold"],
                          channels=ch, x=x, w=w, seed=seed)


def uniform_int8(shape: Sequence[int], seed: int, stream: int = 0,
                 lo: int = -127, hi: int = 127) -> np.ndarray:
    """Uniform int8 values in [lo, hi], for direct GEMM tests."""
    g = _rng(seed, "extra", stream)
    return g.integers(lo, hi + 1, size=tuple(shape), dtype=np.int64).astype(np.int8)


def positive_scales(n: int, seed: int, stream: int = 0) -> np.ndarray:
    """Positive fp32 scale vectors of a realistic spread (about 1e-3 to 1e-1)."""
    g = _rng(seed, "extra", 100 + stream)
    return np.exp(g.uniform(np.log(1e-3), np.log(1e-1), size=n)).astype(np.float32)


def spread_scales(k: int, seed: int, lo_exp: int = -20, hi_exp: int = 20, stream: int = 0) -> np.ndarray:
    """Positive fp32 values with random significands and binary exponents spread
    uniformly over [lo_exp, hi_exp], with edge significands mixed in (1.0,
    all-ones, the lowest and highest exponent), for exercising divisions by
    per-channel factors across their whole range."""
    g = _rng(seed, "extra", 200 + stream)
    mant = g.integers(0, 1 << 23, size=k, dtype=np.int64)
    exps = g.integers(lo_exp, hi_exp + 1, size=k, dtype=np.int64)
    edge = g.choice(k, size=min(k, 64), replace=False)
    mant[edge[0::4]] = 0
    mant[edge[1::4]] = (1 << 23) - 1
    exps[edge[2::4]] = lo_exp
    exps[edge[3::4]] = hi_exp
    bits = ((exps + 127) << 23) | mant
    return bits.astype(np.uint32).view(np.float32)


def cases_for(name: str) -> List[int]:
    return list(CONFIGS[name].get("ms", [CONFIGS[name]["m"]]))
