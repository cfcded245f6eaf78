"""Helpers of the GPU parity tests: device transfer, ulp distances, logging."""
from __future__ import annotations

import sys

import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Exactly representable fp32 numpy values -> a GPU tensor of storage type ``dtype``."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(TORCH_DT[dtype]).to(dev())


def padded(a: np.ndarray, dtype: str, ld: int) -> torch.Tensor:
    """A [rows x cols] view with leading dimension ``ld`` (> cols) on the GPU."""
    rows, cols = a.shape
    full = torch.zeros((rows, ld), dtype=TORCH_DT[dtype])
    full[:, :cols] = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(TORCH_DT[dtype])
    return full.to(dev())[:, :cols]


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp16 tensor -> uint16 bit patterns."""
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


def ordered16(b: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns to integers whose difference counts ulps (+0 == -0)."""
    b = np.asarray(b, np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ordered32(a: np.ndarray) -> np.ndarray:
    b = np.asarray(a, np.float32).view(np.uint32).astype(np.int64)
    mag = b & 0x7FFFFFFF
    return np.where(b & 0x80000000, -mag, mag)


def ulp_diff16(got_bits: np.ndarray, ref_bits: np.ndarray) -> np.ndarray:
    return np.abs(ordered16(got_bits) - ordered16(ref_bits))


def ulp_diff32(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    return np.abs(ordered32(got) - ordered32(ref))


def log(*args):
    print("[gpu-test]", *args, flush=True)
    sys.stdout.flush()


def assert_out_close(y_gpu: torch.Tensor, y_ref: np.ndarray, out: str, what: str = "y") -> float:
    """Output parity: within 1 ulp of the oracle in the output type, zero where it is zero.

    Returns the fraction of bit-exact elements (reported by the callers).
    """
    if out == "f32":
        g = host(y_gpu)
        d = ulp_diff32(g, y_ref)
        zero_ok = np.all(g[y_ref == 0] == 0)
    else:
        g = bits16(y_gpu)
        ref = y_ref.view(np.uint16) if y_ref.dtype != np.uint16 else y_ref
        d = ulp_diff16(g, ref)
        zero_ok = np.all(ordered16(g)[ordered16(ref) == 0] == 0)
    assert d.max(initial=0) <= 1, f"{what}: max ulp difference {d.max()}"
    assert zero_ok, f"{what}: non-zero output where the oracle gives zero"
    return float((d == 0).mean()) if d.size else 1.0
