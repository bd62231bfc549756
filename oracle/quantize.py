"""Quantizers that turn float32 weights into NVFP4 / FP8 codes (test-only oracle).

The pages serve an already-quantized published checkpoint ([P3] "v1.0 got us
here. v1.1 removes its last compromise.": FP4 regions stay FP4, FP8 regions
stay FP8) and never say how it was quantized. Synthetic weights need a
recipe; the plainest one that matches the two formats is used, with every
step in float32 (correctly rounded IEEE), in this order:

NVFP4 (two-level scaling):
  1. s_t = amax(|W|) / (6 * 448), replaced by 1 when that is zero;
  2. per 16-element block b of a row (along K):
     sc = E4M3( (amax_b / 6) / s_t ),  s_b = value(sc);
  3. d = s_b * s_t (one float32 multiply);
  4. if d == 0 every code of the block is the signed zero of its input,
     else c = E2M1( w / d ) (float32 division, then the nearest-even encoder
     of ``formats``, which saturates at 6).

FP8:
  1. s_n = amax(|W[n, :]|) / 448 per output row, replaced by 1 when zero;
  2. c = E4M3( w / s_n ) (float32 division).

Inputs must be finite (an error otherwise).
"""

import numpy as np

from .formats import E2M1_MAX, E4M3_MAX, encode_e2m1, encode_e4m3, decode_e4m3

BLOCK = 16


def _check(w):
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("weights must be a 2-D [N, K] array")
    if not np.isfinite(w).all():
        raise ValueError("weights must be finite")
    return w


def nvfp4_tensor_scale(amax):
    """s_t = amax / 2688 in float32 (1 when that is zero)."""
    s = np.float32(amax) / np.float32(E2M1_MAX * E4M3_MAX)
    return np.float32(1.0) if s == 0 else np.float32(s)


def quantize_nvfp4(w, tensor_scale=None):
    """Quantize float32 W[N, K] (K a multiple of 16) to NVFP4.

    Returns (codes uint8 [N, K] one E2M1 code per element, block_scales uint8
    [N, K/16] E4M3 codes, tensor_scale float32). ``tensor_scale`` overrides
    step 1, so that a subset of rows can be quantized exactly as it would be
    inside the whole tensor.
    """
    w = _check(w)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16")
    if tensor_scale is None:
        s_t = nvfp4_tensor_scale(np.abs(w).max() if w.size else 0.0)
    else:
        s_t = np.float32(tensor_scale)
    blocks = w.reshape(n, k // BLOCK, BLOCK)
    amax_b = np.abs(blocks).max(axis=2) if w.size else np.zeros((n, 0), np.float32)
    ratio = (amax_b / np.float32(E2M1_MAX)) / s_t
    sc = encode_e4m3(ratio)
    s_b = decode_e4m3(sc).astype(np.float32)
    d = s_b * s_t
    zero = d == 0
    safe_d = np.where(zero, np.float32(1.0), d).astype(np.float32)
    q = blocks / safe_d[:, :, None]
    codes = encode_e2m1(q)
    sign_only = (np.signbit(blocks).astype(np.uint8) << 3)
    codes = np.where(zero[:, :, None], sign_only, codes).astype(np.uint8)
    return codes.reshape(n, k), sc.astype(np.uint8), np.float32(s_t)


def quantize_fp8(w):
    """Quantize float32 W[N, K] to E4M3 codes with one fp32 scale per row.

    Returns (codes uint8 [N, K], row_scales float32 [N]).
    """
    w = _check(w)
    amax_r = np.abs(w).max(axis=1) if w.shape[1] else np.zeros(w.shape[0], np.float32)
    s_n = (amax_r / np.float32(E4M3_MAX)).astype(np.float32)
    s_n = np.where(s_n == 0, np.float32(1.0), s_n).astype(np.float32)
    q = w / s_n[:, None]
    return encode_e4m3(q), s_n
