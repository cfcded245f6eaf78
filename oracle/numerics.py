"""Storage-format rounding for the CPU oracle (test infrastructure only).

bf16 is the upper half of an IEEE binary32 word. Rounding a binary32 value to
bf16 with round-to-nearest-even keeps the upper 16 bits after adding
0x7FFF plus the lowest kept bit; that is the textbook RNE on the 16 discarded
bits. NaN and infinities are outside the oracle's contract.

fp16 rounding uses numpy's binary32 -> binary16 cast, which is IEEE
round-to-nearest-even (including the subnormal range).
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact binary32 value."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """binary32 -> nearest bf16 value, returned as binary32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def round_f16(x: np.ndarray) -> np.ndarray:
    """binary32 -> nearest binary16 value, returned as binary16."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def round_to(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a binary32 array to the storage type ``dtype`` ('f32', 'bf16', 'f16').

    Returns binary32 for 'f32', uint16 bf16 bit patterns for 'bf16' and
    numpy float16 for 'f16'.
    """
    if dtype == "f32":
        return np.asarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f16":
        return round_f16(x32)
    raise ValueError(dtype)
