"""SmoothQuant W8A8 int8 linear layer for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/sq.h`` (``libsq.so``, built
in-tree by ``w8a8_int8_quantization_amd.build``). Each ``sq_*`` function here
carries the name of the C entry point it calls: it checks that the tensors are
on the GPU, allocates outputs with torch, passes raw device pointers and the
current HIP stream, and raises :class:`SQError` on a non-zero status. All the
arithmetic runs in the HIP kernels; there is no fallback of any kind, and
importing this package fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "SQError", "lib_path", "sq_version",
    "sq_calibrate_absmax", "sq_smooth_fold_weights", "sq_quant_act_per_token", "sq_w8a8_linear",
    "sq_w8a8_linear_dyn", "sq_outlier_detect", "sq_quant_act_rows_masked", "sq_int8_decomp_linear",
    "sq_int8_decomp_gemm", "linear_workspace", "sq_fold_norm_gain", "sq_rmsnorm_quant", "sq_rmsnorm_w8a8_linear",
    "sq_silu_mul_quant", "sq_silu_mul_w8a8_linear", "sq_quant_act_fp8", "sq_quant_weights_fp8", "sq_fp8_linear",
    "sq_fp8_linear_dyn", "fp8_linear_workspace", "sq_gptq_hessian", "sq_gptq_quantize", "MAX_K_GPTQ",
    "SMOOTH_COMPUTE", "SMOOTH_GIVEN", "SMOOTH_NONE", "MAX_K_INT32", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# SQ_LIBRARY selects another build of the same library (the host-sanitized
# one that the CPU tests load); by default the in-tree libsq.so.
lib_path = os.environ.get("SQ_LIBRARY") or os.path.join(_PKG, "libsq.so")

if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is missing: the HIP library has not been built. "
        "Run `python w8a8_int8_quantization_amd/build.py` (or __graft_entry__.build()).")

_lib = ctypes.CDLL(lib_path)

SQ_F32, SQ_BF16, SQ_F16, SQ_I32, SQ_I8 = 0, 1, 2, 3, 4
SMOOTH_COMPUTE, SMOOTH_GIVEN, SMOOTH_NONE = 0, 1, 2
MAX_K_INT32 = 133144
MAX_K_GPTQ = 32768

_i64, _u32, _sz, _p, _f, _d = ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, \
    ctypes.c_double
_st = ctypes.c_int

# name -> (restype, argtypes), exactly as declared in include/sq.h
_SIGS = {
    "sq_status_string": (ctypes.c_char_p, [_st]),
    "sq_last_hip_error": (ctypes.c_int, []),
    "sq_version": (ctypes.c_int, []),
    "sq_calibrate_absmax": (_st, [_p, _st, _i64, _i64, _i64, _p, _p]),
    "sq_smooth_fold_workspace_size": (_sz, [_i64, _i64]),
    "sq_smooth_fold_weights": (_st, [_p, _p, _st, _i64, _i64, _i64, _d, _u32, _p, _p, _p, _p, _sz, _p]),
    "sq_quant_act_per_token": (_st, [_p, _st, _i64, _i64, _i64, _p, _p, _p, _p]),
    "sq_w8a8_linear_workspace_size": (_sz, [_i64, _i64, _i64]),
    "sq_w8a8_linear": (_st, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _st, _i64, _p, _sz, _p]),
    "sq_w8a8_linear_dyn_workspace_size": (_sz, [_i64, _i64, _i64]),
    "sq_w8a8_linear_dyn": (_st, [_p, _st, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _st, _i64, _p, _sz, _p]),
    "sq_w8a8_linear_dyn_static": (_st, [_p, _st, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _st, _i64, _p]),
    "sq_fold_norm_gain": (_st, [_p, _st, _p, _i64, _p, _p]),
    "sq_rmsnorm_quant": (_st, [_p, _st, _i64, _i64, _i64, _p, _f, _p, _p, _p]),
    "sq_rmsnorm_w8a8_linear_workspace_size": (_sz, [_i64, _i64, _i64]),
    "sq_rmsnorm_w8a8_linear": (_st, [_p, _st, _i64, _p, _f, _p, _p, _i64, _i64, _i64, _p, _st, _i64, _p, _sz, _p]),
    "sq_silu_mul_quant": (_st, [_p, _p, _st, _i64, _i64, _i64, _i64, _p, _p, _p, _p]),
    "sq_silu_mul_w8a8_linear_workspace_size": (_sz, [_i64, _i64, _i64]),
    "sq_silu_mul_w8a8_linear": (_st, [_p, _p, _st, _i64, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _st, _i64, _p, _sz,
                                      _p]),
    "sq_quant_act_fp8": (_st, [_p, _st, _i64, _i64, _i64, _p, _p, _p]),
    "sq_quant_weights_fp8_workspace_size": (_sz, [_i64, _i64]),
    "sq_quant_weights_fp8": (_st, [_p, _st, _i64, _i64, _i64, _p, _p, _p, _sz, _p]),
    "sq_fp8_linear_workspace_size": (_sz, [_i64, _i64, _i64]),
    "sq_fp8_linear": (_st, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _st, _i64, _p, _sz, _p]),
    "sq_fp8_linear_dyn_workspace_size": (_sz, [_i64, _i64, _i64]),
    "sq_gptq_hessian": (_st, [_p, _st, _i64, _i64, _i64, _p, _p, _p]),
    "sq_gptq_quantize_workspace_size": (_sz, [_i64, _i64]),
    "sq_gptq_quantize": (_st, [_p, _p, _st, _i64, _i64, _i64, _p, _f, _p, _p, _p, _sz, _p]),
    "sq_fp8_linear_dyn": (_st, [_p, _st, _i64, _p, _p, _i64, _i64, _i64, _p, _st, _i64, _p, _sz, _p]),
    "sq_outlier_detect_workspace_size": (_sz, [_i64]),
    "sq_outlier_detect": (_st, [_p, _st, _i64, _i64, _i64, _f, _p, _p, _p, _p, _sz, _p]),
    "sq_quant_act_rows_masked": (_st, [_p, _st, _i64, _i64, _i64, _p, _p, _p, _p]),
    "sq_int8_decomp_workspace_size": (_sz, [_i64, _i64, _i64]),
    "sq_int8_decomp_gemm": (_st, [_p, _p, _p, _i64, _p, _p, _p, _i64, _p, _p, _i64, _i64, _i64, _p, _i64, _p]),
    "sq_int8_decomp_linear": (_st, [_p, _i64, _p, _p, _p, _i64, _i64, _i64, _i64, _f, _p, _i64, _p, _p, _sz, _p]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

raw = {}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args
    raw[_name] = _fn


class SQError(RuntimeError):
    def __init__(self, call: str, status: int):
        msg = raw["sq_status_string"](status).decode()
        if status == 7:
            msg += f" (hipError {raw['sq_last_hip_error']()})"
        super().__init__(f"{call}: status {status}: {msg}")
        self.status = status


def _check(call: str, status: int) -> None:
    if status != 0:
        raise SQError(call, status)


_DT = {torch.float32: SQ_F32, torch.bfloat16: SQ_BF16, torch.float16: SQ_F16, torch.int32: SQ_I32}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return t.data_ptr()


def _rows(t: torch.Tensor) -> Tuple[int, int, int]:
    """(rows, cols, leading dimension) of a 2-D tensor with unit column stride."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D row-major tensor")
    return t.shape[0], t.shape[1], max(t.stride(0), t.shape[1])


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def linear_workspace(m: int, n: int, k: int, device) -> Optional[torch.Tensor]:
    """A zero-filled workspace for ``sq_w8a8_linear`` at this shape (None if it needs none).

    Reusable across calls at the same shape: each call restores its counter
    words to zero (the rest is scratch that every call writes before reading)."""
    nb = raw["sq_w8a8_linear_workspace_size"](m, n, k)
    return torch.zeros(nb, dtype=torch.uint8, device=device) if nb else None


def sq_version() -> int:
    return raw["sq_version"]()


def sq_calibrate_absmax(x: torch.Tensor, absmax: torch.Tensor) -> torch.Tensor:
    """Running per-channel max |x| over the rows of ``x``, in place into ``absmax`` [K] fp32."""
    t, k, ldx = _rows(x)
    _check("sq_calibrate_absmax", raw["sq_calibrate_absmax"](_ptr(x), _dt(x), t, k, ldx, _ptr(absmax),
                                                             _stream(x.device)))
    return absmax


def sq_smooth_fold_weights(w: torch.Tensor, alpha: float = 0.5, absmax: Optional[torch.Tensor] = None,
                           smooth: Optional[torch.Tensor] = None, flags: int = SMOOTH_COMPUTE):
    """Smoothing factors, fold and per-channel int8 quantisation of W [K x N].

    Returns (smooth [K] fp32 or None, wq [N x K] int8, w_scale [N] fp32).
    """
    k, n, ldw = _rows(w)
    dev = w.device
    if flags == SMOOTH_COMPUTE and smooth is None:
        smooth = torch.empty(k, dtype=torch.float32, device=dev)
    wq = torch.empty((n, k), dtype=torch.int8, device=dev)
    w_scale = torch.empty(n, dtype=torch.float32, device=dev)
    nb = raw["sq_smooth_fold_workspace_size"](k, n)
    ws = _workspace(nb, dev)
    _check("sq_smooth_fold_weights", raw["sq_smooth_fold_weights"](
        _ptr(absmax), _ptr(w), _dt(w), k, n, ldw, float(alpha), flags, _ptr(smooth), _ptr(wq), _ptr(w_scale),
        _ptr(ws), nb, _stream(dev)))
    return smooth, wq, w_scale


def sq_quant_act_per_token(x: torch.Tensor, smooth: Optional[torch.Tensor] = None,
                           xq: Optional[torch.Tensor] = None, x_scale: Optional[torch.Tensor] = None):
    """Per-token int8 quantisation of X [M x K] (divided by ``smooth`` first if given)."""
    m, k, ldx = _rows(x)
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device) if xq is None else xq
    x_scale = torch.empty(m, dtype=torch.float32, device=x.device) if x_scale is None else x_scale
    _check("sq_quant_act_per_token", raw["sq_quant_act_per_token"](
        _ptr(x), _dt(x), m, k, ldx, _ptr(smooth), _ptr(xq), _ptr(x_scale), _stream(x.device)))
    return xq, x_scale


def sq_w8a8_linear(xq: torch.Tensor, x_scale: Optional[torch.Tensor], wq: torch.Tensor,
                   w_scale: Optional[torch.Tensor], out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None):
    """int8 GEMM with the fused dequantisation; out_dtype torch.int32 returns the raw accumulator.

    ``ws``: a workspace from :func:`linear_workspace` (zero-filled, reusable at
    this shape); a fresh one is allocated when None."""
    m, k, _ = _rows(xq)
    n = wq.shape[0]
    if wq.shape[1] != k:
        raise ValueError("xq and wq disagree on K")
    y = torch.empty((m, n), dtype=out_dtype, device=xq.device) if y is None else y
    _, _, ldy = _rows(y)
    if ws is None:
        ws = linear_workspace(m, n, k, xq.device)
    _check("sq_w8a8_linear", raw["sq_w8a8_linear"](
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), m, n, k, _ptr(y), _dt(y), ldy, _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(xq.device)))
    return y


def sq_w8a8_linear_dyn(x: torch.Tensor, smooth: Optional[torch.Tensor], wq: torch.Tensor, w_scale: torch.Tensor,
                       out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None):
    """Per-token quantisation and the W8A8 GEMM in one call."""
    m, k, ldx = _rows(x)
    n = wq.shape[0]
    y = torch.empty((m, n), dtype=out_dtype, device=x.device) if y is None else y
    _, _, ldy = _rows(y)
    nb = raw["sq_w8a8_linear_dyn_workspace_size"](m, n, k)
    if ws is None:
        ws = _workspace(nb, x.device)
    _check("sq_w8a8_linear_dyn", raw["sq_w8a8_linear_dyn"](
        _ptr(x), _dt(x), ldx, _ptr(smooth), _ptr(wq), _ptr(w_scale), m, n, k, _ptr(y), _dt(y), ldy,
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(x.device)))
    return y


def sq_w8a8_linear_dyn_static(x: torch.Tensor, smooth: Optional[torch.Tensor], wq: torch.Tensor,
                              w_scale: torch.Tensor, out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None):
    """:func:`sq_w8a8_linear_dyn` with the library's static scratch instead of a workspace."""
    m, k, ldx = _rows(x)
    n = wq.shape[0]
    y = torch.empty((m, n), dtype=out_dtype, device=x.device) if y is None else y
    _, _, ldy = _rows(y)
    _check("sq_w8a8_linear_dyn_static", raw["sq_w8a8_linear_dyn_static"](
        _ptr(x), _dt(x), ldx, _ptr(smooth), _ptr(wq), _ptr(w_scale), m, n, k, _ptr(y), _dt(y), ldy,
        _stream(x.device)))
    return y


def sq_fold_norm_gain(gamma: torch.Tensor, smooth: Optional[torch.Tensor] = None,
                      gain: Optional[torch.Tensor] = None) -> torch.Tensor:
    """RMSNorm gain with the smoothing factor folded in: gamma / s (binary32 [K])."""
    k = gamma.numel()
    gain = torch.empty(k, dtype=torch.float32, device=gamma.device) if gain is None else gain
    _check("sq_fold_norm_gain", raw["sq_fold_norm_gain"](
        _ptr(gamma), _dt(gamma), _ptr(smooth), k, _ptr(gain), _stream(gamma.device)))
    return gain


def sq_rmsnorm_quant(x: torch.Tensor, gain: torch.Tensor, eps: float = 0.0,
                     xq: Optional[torch.Tensor] = None, x_scale: Optional[torch.Tensor] = None):
    """RMSNorm of X [M x K] with the folded gain, then per-token int8 quantisation."""
    m, k, ldx = _rows(x)
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device) if xq is None else xq
    x_scale = torch.empty(m, dtype=torch.float32, device=x.device) if x_scale is None else x_scale
    _check("sq_rmsnorm_quant", raw["sq_rmsnorm_quant"](
        _ptr(x), _dt(x), m, k, ldx, _ptr(gain), float(eps), _ptr(xq), _ptr(x_scale), _stream(x.device)))
    return xq, x_scale


def sq_rmsnorm_w8a8_linear(x: torch.Tensor, gain: torch.Tensor, eps: float, wq: torch.Tensor,
                           w_scale: torch.Tensor, out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None):
    """RMSNorm with the folded gain, per-token quantisation and the W8A8 GEMM in one call."""
    m, k, ldx = _rows(x)
    n = wq.shape[0]
    y = torch.empty((m, n), dtype=out_dtype, device=x.device) if y is None else y
    _, _, ldy = _rows(y)
    nb = raw["sq_rmsnorm_w8a8_linear_workspace_size"](m, n, k)
    if ws is None:
        ws = _workspace(nb, x.device)
    _check("sq_rmsnorm_w8a8_linear", raw["sq_rmsnorm_w8a8_linear"](
        _ptr(x), _dt(x), ldx, _ptr(gain), float(eps), _ptr(wq), _ptr(w_scale), m, n, k, _ptr(y), _dt(y), ldy,
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(x.device)))
    return y


def sq_silu_mul_quant(gate: torch.Tensor, up: torch.Tensor, smooth: Optional[torch.Tensor] = None,
                      xq: Optional[torch.Tensor] = None, x_scale: Optional[torch.Tensor] = None):
    """h = SiLU(gate) * up (bf16 [M x K] each), divided by ``smooth`` and quantised per token."""
    m, k, ldg = _rows(gate)
    mu, ku, ldu = _rows(up)
    if (mu, ku) != (m, k):
        raise ValueError("gate and up differ in shape")
    xq = torch.empty((m, k), dtype=torch.int8, device=gate.device) if xq is None else xq
    x_scale = torch.empty(m, dtype=torch.float32, device=gate.device) if x_scale is None else x_scale
    _check("sq_silu_mul_quant", raw["sq_silu_mul_quant"](
        _ptr(gate), _ptr(up), _dt(gate), m, k, ldg, ldu, _ptr(smooth), _ptr(xq), _ptr(x_scale),
        _stream(gate.device)))
    return xq, x_scale


def sq_silu_mul_w8a8_linear(gate: torch.Tensor, up: torch.Tensor, smooth: Optional[torch.Tensor], wq: torch.Tensor,
                            w_scale: torch.Tensor, out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None):
    """SiLU(gate) * up, smoothing, per-token quantisation and the W8A8 GEMM in one call."""
    m, k, ldg = _rows(gate)
    _, _, ldu = _rows(up)
    n = wq.shape[0]
    y = torch.empty((m, n), dtype=out_dtype, device=gate.device) if y is None else y
    _, _, ldy = _rows(y)
    nb = raw["sq_silu_mul_w8a8_linear_workspace_size"](m, n, k)
    if ws is None:
        ws = _workspace(nb, gate.device)
    _check("sq_silu_mul_w8a8_linear", raw["sq_silu_mul_w8a8_linear"](
        _ptr(gate), _ptr(up), _dt(gate), ldg, ldu, _ptr(smooth), _ptr(wq), _ptr(w_scale), m, n, k, _ptr(y), _dt(y),
        ldy, _ptr(ws), ws.numel() if ws is not None else 0, _stream(gate.device)))
    return y


def sq_quant_act_fp8(x: torch.Tensor, xq: Optional[torch.Tensor] = None, x_scale: Optional[torch.Tensor] = None):
    """Per-token E4M3 quantisation of X [M x K]: (codes uint8 [M x K], scales [M])."""
    m, k, ldx = _rows(x)
    xq = torch.empty((m, k), dtype=torch.uint8, device=x.device) if xq is None else xq
    x_scale = torch.empty(m, dtype=torch.float32, device=x.device) if x_scale is None else x_scale
    _check("sq_quant_act_fp8", raw["sq_quant_act_fp8"](
        _ptr(x), _dt(x), m, k, ldx, _ptr(xq), _ptr(x_scale), _stream(x.device)))
    return xq, x_scale


def sq_quant_weights_fp8(w: torch.Tensor):
    """Per-output-channel E4M3 quantisation of W [K x N]: (codes uint8 [N x K], scales [N])."""
    k, n, ldw = _rows(w)
    wq = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    w_scale = torch.empty(n, dtype=torch.float32, device=w.device)
    nb = raw["sq_quant_weights_fp8_workspace_size"](k, n)
    ws = _workspace(nb, w.device)
    _check("sq_quant_weights_fp8", raw["sq_quant_weights_fp8"](
        _ptr(w), _dt(w), k, n, ldw, _ptr(wq), _ptr(w_scale), _ptr(ws), nb, _stream(w.device)))
    return wq, w_scale


def fp8_linear_workspace(m: int, n: int, k: int, device) -> Optional[torch.Tensor]:
    """A zero-filled workspace for ``sq_fp8_linear`` at this shape (None if it needs none);
    reusable across calls at the same shape."""
    nb = raw["sq_fp8_linear_workspace_size"](m, n, k)
    return torch.zeros(nb, dtype=torch.uint8, device=device) if nb else None


def sq_fp8_linear(xq: torch.Tensor, x_scale: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                  out_dtype=torch.bfloat16, y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """E4M3 GEMM on the matrix cores with the per-token x per-channel dequantisation.

    ``ws``: a workspace from :func:`fp8_linear_workspace`; a fresh one is allocated when None."""
    m, k, _ = _rows(xq)
    n = wq.shape[0]
    y = torch.empty((m, n), dtype=out_dtype, device=xq.device) if y is None else y
    _, _, ldy = _rows(y)
    if ws is None:
        ws = fp8_linear_workspace(m, n, k, xq.device)
    _check("sq_fp8_linear", raw["sq_fp8_linear"](
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), m, n, k, _ptr(y), _dt(y), ldy, _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(xq.device)))
    return y


def sq_fp8_linear_dyn(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, out_dtype=torch.bfloat16,
                      y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Per-token E4M3 quantisation and the E4M3 GEMM in one call."""
    m, k, ldx = _rows(x)
    n = wq.shape[0]
    y = torch.empty((m, n), dtype=out_dtype, device=x.device) if y is None else y
    _, _, ldy = _rows(y)
    nb = raw["sq_fp8_linear_dyn_workspace_size"](m, n, k)
    if ws is None:
        ws = _workspace(nb, x.device)
    _check("sq_fp8_linear_dyn", raw["sq_fp8_linear_dyn"](
        _ptr(x), _dt(x), ldx, _ptr(wq), _ptr(w_scale), m, n, k, _ptr(y), _dt(y), ldy, _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(x.device)))
    return y


def sq_gptq_hessian(x: torch.Tensor, smooth: Optional[torch.Tensor] = None, h: Optional[torch.Tensor] = None):
    """h += Xh^T Xh over the calibration rows x (Xh = fl32(x / smooth)), binary64 [K x K];
    a zero-filled h is allocated when None. Returns h."""
    t, k, ldx = _rows(x)
    h = torch.zeros((k, k), dtype=torch.float64, device=x.device) if h is None else h
    _check("sq_gptq_hessian", raw["sq_gptq_hessian"](
        _ptr(x), _dt(x), t, k, ldx, _ptr(smooth), _ptr(h), _stream(x.device)))
    return h


def sq_gptq_quantize(h: torch.Tensor, w: torch.Tensor, smooth: Optional[torch.Tensor] = None, damp: float = 0.01,
                     ws: Optional[torch.Tensor] = None):
    """GPTQ of W [K x N] (smoothed by s when given) against h: (Wq [N x K] int8, w_scale [N])."""
    k, n, ldw = _rows(w)
    wq = torch.empty((n, k), dtype=torch.int8, device=w.device)
    w_scale = torch.empty(n, dtype=torch.float32, device=w.device)
    nb = raw["sq_gptq_quantize_workspace_size"](k, n)
    if ws is None:
        ws = _workspace(nb, w.device)
    _check("sq_gptq_quantize", raw["sq_gptq_quantize"](
        _ptr(h), _ptr(w), _dt(w), k, n, ldw, _ptr(smooth), float(damp), _ptr(wq), _ptr(w_scale), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(w.device)))
    return wq, w_scale


def sq_outlier_detect(x: torch.Tensor, threshold: float = 6.0):
    """(mask [K] uint8, idx [K] int32 of which the first ``count`` are defined, count [1] int32)."""
    m, k, ldx = _rows(x)
    dev = x.device
    mask = torch.empty(k, dtype=torch.uint8, device=dev)
    idx = torch.empty(k, dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int32, device=dev)
    nb = raw["sq_outlier_detect_workspace_size"](k)
    ws = _workspace(nb, dev)
    _check("sq_outlier_detect", raw["sq_outlier_detect"](
        _ptr(x), _dt(x), m, k, ldx, float(threshold), _ptr(mask), _ptr(idx), _ptr(count), _ptr(ws), nb,
        _stream(dev)))
    return mask, idx, count


def sq_quant_act_rows_masked(x: torch.Tensor, mask: torch.Tensor):
    """Row-wise int8 over the columns where ``mask`` is 0; masked columns of Xq are 0."""
    m, k, ldx = _rows(x)
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    x_scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("sq_quant_act_rows_masked", raw["sq_quant_act_rows_masked"](
        _ptr(x), _dt(x), m, k, ldx, _ptr(mask), _ptr(xq), _ptr(x_scale), _stream(x.device)))
    return xq, x_scale


def sq_int8_decomp_linear(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, w16: torch.Tensor,
                          threshold: float = 6.0, y: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None):
    """LLM.int8() decomposed linear layer (fp16). Returns (y [M x N] fp16, n_outliers [1] int32)."""
    m, k, ldx = _rows(x)
    n = wq.shape[0]
    _, _, ldw = _rows(w16)
    y = torch.empty((m, n), dtype=torch.float16, device=x.device) if y is None else y
    _, _, ldy = _rows(y)
    cnt = torch.empty(1, dtype=torch.int32, device=x.device)
    nb = raw["sq_int8_decomp_workspace_size"](m, n, k)
    if ws is None:
        ws = _workspace(nb, x.device)
    _check("sq_int8_decomp_linear", raw["sq_int8_decomp_linear"](
        _ptr(x), ldx, _ptr(wq), _ptr(w_scale), _ptr(w16), ldw, m, n, k, float(threshold), _ptr(y), ldy,
        _ptr(cnt), _ptr(ws), ws.numel() if ws is not None else 0, _stream(x.device)))
    return y, cnt


def sq_int8_decomp_gemm(xq: torch.Tensor, x_scale: torch.Tensor, x: torch.Tensor, wq: torch.Tensor,
                        w_scale: torch.Tensor, w16: torch.Tensor, idx: torch.Tensor, count: torch.Tensor,
                        y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 GEMM of the masked quantised X plus the fp16 outlier slice (LLM.int8() second half)."""
    m, k, _ = _rows(xq)
    _, _, ldx = _rows(x)
    n = wq.shape[0]
    _, _, ldw = _rows(w16)
    y = torch.empty((m, n), dtype=torch.float16, device=xq.device) if y is None else y
    _, _, ldy = _rows(y)
    _check("sq_int8_decomp_gemm", raw["sq_int8_decomp_gemm"](
        _ptr(xq), _ptr(x_scale), _ptr(x), ldx, _ptr(wq), _ptr(w_scale), _ptr(w16), ldw, _ptr(idx), _ptr(count),
        m, n, k, _ptr(y), ldy, _stream(xq.device)))
    return y
