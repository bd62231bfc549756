"""Canonical byte layout of NVFP4 codes (test-only oracle).

The pages do not say how two 4-bit codes share a byte. Reading used here
(the common convention for packed FP4 tensors): row-major [N][K/2] bytes,
element 2j of a row in the LOW nibble of byte j and element 2j+1 in the HIGH
nibble. Block scales are row-major [N][K/16] bytes (one E4M3 code each) and
FP8 codes are row-major [N][K] bytes; neither needs any packing.
"""

import numpy as np


def pack_nibbles(codes):
    """uint8 [N, K] of 4-bit codes -> uint8 [N, K/2] (even element low)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("K must be even")
    if codes.size and int(codes.max()) > 15:
        raise ValueError("codes must be 0..15")
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """uint8 [N, K/2] -> uint8 [N, K] of 4-bit codes (inverse of pack)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out
