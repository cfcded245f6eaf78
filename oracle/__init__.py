"""CPU oracle for the SmoothQuant W8A8 linear layer, the RMSNorm that carries its
smoothing factor, the gated activation feeding the down projection, GPTQ weight
rounding, the FP8 (E4M3) variant and the LLM.int8() variant.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition of what the HIP path computes; it exists to check that path. Only
the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it. It shares no code, constant or helper with the
HIP library or its Python binding, and imports neither.

Every function is pinned by CPU tests to values the pages print (worked
examples, corrected where their arithmetic slips), closed forms, invariants
and brute force; none is marked "parity unpinned".
"""
from .numerics import f32_to_bf16_bits, bf16_bits_to_f32, round_bf16, round_f16, round_to
from .smoothquant import (
    QMAX,
    calibrate_absmax,
    weight_row_absmax,
    smoothing_factors,
    fold_weights,
    quantize_weights_per_channel,
    smooth_fold_quantize,
    smooth_activations,
    quantize_activations,
    int8_matmul,
    dequantize,
    w8a8_linear,
    smoothquant_linear,
    per_tensor_int8_linear,
)
from .llm_int8 import detect_outliers, quantize_rows_regular, fp16_outlier_product, int8_decomp_linear
from .rmsnorm import fold_norm_gain, rms_inverse, apply_gain, rmsnorm, rmsnorm_quantize
from .silu import exp32, silu32, gated_activation, silu_mul_quantize
from .fp8 import (e4m3_values, e4m3_encode, e4m3_decode, quantize_activations_fp8, quantize_weights_fp8,
                  fp8_matmul, fp8_linear)
from .gptq import GPTQ_DAMP, gptq_hessian, gptq_quantize, gptq_smooth_quantize

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "round_bf16", "round_f16", "round_to",
    "QMAX", "calibrate_absmax", "weight_row_absmax", "smoothing_factors", "fold_weights",
    "quantize_weights_per_channel", "smooth_fold_quantize", "smooth_activations",
    "quantize_activations", "int8_matmul", "dequantize", "w8a8_linear", "smoothquant_linear",
    "per_tensor_int8_linear", "detect_outliers", "quantize_rows_regular",
    "fp16_outlier_product", "int8_decomp_linear", "fold_norm_gain", "rms_inverse", "apply_gain", "rmsnorm",
    "rmsnorm_quantize", "exp32", "silu32", "gated_activation", "silu_mul_quantize", "e4m3_values", "e4m3_encode",
    "e4m3_decode", "quantize_activations_fp8", "quantize_weights_fp8", "fp8_matmul", "fp8_linear",
    "GPTQ_DAMP", "gptq_hessian", "gptq_quantize", "gptq_smooth_quantize",
]
