"""Dequantize-then-matmul in float64: the result the skinny GEMM must reach.

[P3] "What I actually built": the kernel keeps the weights compressed while
they stream from HBM and converts each fragment to FP16 right before the
matrix multiply, with no dequantize-to-FP16 pass over the model. Whatever
order it takes, the value it approximates is the plain product of the FP16
activation rows with the dequantized weights:

    y[m, n] = sum_k x[m, k] * wdq[n, k]
    NVFP4:  wdq[n, k] = E2M1(c[n, k]) * E4M3(s[n, k // 16]) * s_t
    FP8:    wdq[n, k] = E4M3(c[n, k]) * s_n[n]

M is the number of activation rows: 1 for plain decode, up to 8 for a k=7
speculative verify round (the current token plus seven drafts; [P3] "What I
actually built", the paragraph on the eight-row tile).

Every product here is exact in float64 (an fp16 value has 11 significant
bits; E2M1*E4M3 has at most 6 and the fp32 scale 24), and the float64 sum
adds at most K * 2^-53 * sum|x*w| of error, far below the acceptance bound.
Alongside y the oracle returns b[m, n] = sum_k |x[m, k] * wdq[n, k]|, the
scale of the acceptance bound |y_gpu - y| <= 2e-3 * b + 1e-3.
"""

import numpy as np

from .formats import decode_e2m1, decode_e4m3

BLOCK = 16


def dequantize_nvfp4(codes, block_scales, tensor_scale):
    """float64 W[N, K] from E2M1 codes [N, K], E4M3 block scales [N, K/16]
    and the fp32 tensor scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    block_scales = np.asarray(block_scales, dtype=np.uint8)
    n, k = codes.shape
    if block_scales.shape != (n, k // BLOCK) or k % BLOCK:
        raise ValueError("block scales must be [N, K/16]")
    sb = decode_e4m3(block_scales)
    if np.isnan(sb).any():
        raise ValueError("NaN block scale")
    return decode_e2m1(codes) * np.repeat(sb, BLOCK, axis=1) * np.float64(np.float32(tensor_scale))


def dequantize_fp8(codes, row_scales):
    """float64 W[N, K] from E4M3 codes [N, K] and fp32 row scales [N]."""
    w = decode_e4m3(codes)
    if np.isnan(w).any():
        raise ValueError("NaN FP8 code")
    rs = np.asarray(row_scales, dtype=np.float32).astype(np.float64)
    return w * rs[:, None]


def skinny_gemm(x, wdq):
    """(y, b) for fp16 activations x[M, K] and float64 weights wdq[N, K]."""
    xd = np.asarray(x, dtype=np.float16).astype(np.float64)
    wdq = np.asarray(wdq, dtype=np.float64)
    if xd.shape[1] != wdq.shape[1]:
        raise ValueError("x and W disagree on K")
    y = xd @ wdq.T
    b = np.abs(xd) @ np.abs(wdq).T
    return y, b


def gemm_nvfp4(x, codes, block_scales, tensor_scale):
    return skinny_gemm(x, dequantize_nvfp4(codes, block_scales, tensor_scale))


def gemm_fp8(x, codes, row_scales):
    return skinny_gemm(x, dequantize_fp8(codes, row_scales))


def tolerance(b):
    """Per-element acceptance bound 2e-3 * b + 1e-3 for a GEMM output."""
    return 2e-3 * np.asarray(b, dtype=np.float64) + 1e-3


def argmax_candidates(y, b):
    """For each row of a GEMM output, the indices that can be its argmax once
    every element is known only to within the acceptance bound t = tolerance(b):
    i qualifies when y[i] + t[i] >= max_j (y[j] - t[j]). (A greedy decoder
    takes the largest logit; when two logits are closer than the bound, either
    is a correct answer.) Returns a boolean mask of y's shape; each row has at
    least the exact argmax."""
    y = np.asarray(y, dtype=np.float64)
    t = tolerance(b)
    floor = np.max(y - t, axis=-1, keepdims=True)
    return (y + t) >= floor
