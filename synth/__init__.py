"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package holds input preparation only (random draws, 3D token grids,
bf16 rounding, per-tensor e4m3 and block-scaled MX e4m3 quantization of the inputs). It contains none of the attention method's
arithmetic, so that the fp64 oracle and the HIP kernels can both be fed the
same bytes without sharing any computation.
"""
from .video_tokens import (  # noqa: F401
    CONFIGS,
    VideoTokenConfig,
    bf16_bits_to_f32,
    e4m3_bits_to_f32,
    f32_to_bf16_bits,
    e8m0_to_f64,
    f32_to_e4m3_bits,
    make_fp8_inputs,
    make_mxfp8_qk_inputs,
    mxfp8_dequantize,
    quantize_mxfp8_bf16,
    make_inputs,
    quantize_e4m3,
)
