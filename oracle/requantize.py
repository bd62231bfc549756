"""Offline conversion of FP8 weights to NVFP4 (test infrastructure only).

[P3] "v1.0 got us here. v1.1 removes its last compromise.": the first
version of the post's engine served the checkpoint's FP8 regions by
converting them into NVFP4, because the old GPU had no FP8 path; the second
kept them FP8. The pages do not give the conversion's arithmetic. The
plainest reading is taken here: the FP8 weights are dequantized to the fp32
values they stand for (the E4M3 value times the row's fp32 scale, one fp32
multiply, rounded to nearest even) and those values are quantized with the
NVFP4 recipe of ``quantize.quantize_nvfp4`` (tensor scale from their
absolute maximum, an E4M3 scale per 16 elements, E2M1 codes).
"""

import numpy as np

from .formats import decode_e4m3
from .quantize import quantize_nvfp4


def dequantize_fp8_f32(codes, row_scales):
    """fp32 W[N, K] = E4M3(c[n, k]) * s_n, each product rounded once to fp32."""
    v = decode_e4m3(np.asarray(codes, dtype=np.uint8))
    if np.isnan(v).any():
        raise ValueError("NaN FP8 code")
    s = np.asarray(row_scales, dtype=np.float32)
    return v.astype(np.float32) * s[:, None]


def requantize_fp8_to_nvfp4(codes, row_scales):
    """(E2M1 codes [N, K], E4M3 block scales [N, K/16], fp32 tensor scale) of
    the FP8 weight (codes [N, K], fp32 row scales [N])."""
    return quantize_nvfp4(dequantize_fp8_f32(codes, row_scales))
