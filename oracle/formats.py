"""E2M1 and E4M3 tables, decoders and encoders (float64 oracle; test-only).

The pages name the two weight formats without defining them ([P3] "What I
actually built": the NVFP4 path; the FP8 regions of the checkpoint in
[P3] "v1.0 got us here. v1.1 removes its last compromise."). The tables here
are built from the public bit-field definitions:

* E2M1 (OCP Microscaling spec v1.0, FP4 element): bits s|e1 e0|m, exponent
  bias 1. e = 0 is subnormal, value (-1)^s * 0.5 * m; otherwise
  (-1)^s * 2^(e-1) * (1 + m/2). Magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; no
  NaN and no infinity.
* E4M3 "FN" (OCP 8-bit floating point spec): bits s|eeee|mmm, bias 7. e = 0
  is subnormal, value (-1)^s * 2^-6 * m/8; otherwise (-1)^s * 2^(e-7) *
  (1 + m/8). S.1111.111 (0x7F, 0xFF) is NaN; there is no infinity; the
  largest finite magnitude is 448.

Encoders are written as a brute-force search: the code whose value is nearest
to the input, by exact distance. Readings (the pages give none of this):

* ties go to the code whose lowest bit (the lowest mantissa bit) is 0, i.e.
  round-half-to-even;
* the search runs over finite codes only and inputs are clamped to the
  largest finite magnitude first, so out-of-range inputs saturate and
  infinities produced by an earlier fp32 step land on +-max;
* the sign bit is copied from the input, so -0.0 and negative inputs that
  round to zero give the negative-zero code;
* NaN inputs are an error.

Exactness of the search: inputs are float32 and table entries carry at most
4 significant bits, so |v - t| is exact in float64 whenever v is within
2^40 of t; when it is not, v is far from every rounding boundary and
rounding of the distances cannot change which entry is nearest.
"""

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0

_CHUNK = 1 << 15


def e2m1_table():
    """Value of each of the 16 E2M1 codes, from the bit fields (float64)."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        s = (code >> 3) & 1
        e = (code >> 1) & 3
        m = code & 1
        if e == 0:
            mag = 0.5 * m
        else:
            mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
        vals[code] = -mag if s else mag
    return vals


def e4m3_table():
    """Value of each of the 256 E4M3FN codes, from the bit fields (float64).

    0x7F and 0xFF are NaN.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 15
        m = code & 7
        if e == 15 and m == 7:
            vals[code] = np.nan
            continue
        if e == 0:
            mag = 2.0 ** -6 * (m / 8.0)
        else:
            mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
        vals[code] = -mag if s else mag
    return vals


_E2M1 = e2m1_table()
_E4M3 = e4m3_table()


def decode_e2m1(codes):
    """float64 values of an array of E2M1 codes (uint8, each 0..15)."""
    codes = np.asarray(codes)
    if codes.size and int(codes.max()) > 15:
        raise ValueError("E2M1 codes must be 0..15")
    return _E2M1[codes.astype(np.intp)]


def decode_e4m3(codes):
    """float64 values of an array of E4M3FN codes (uint8); NaN codes give NaN."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _E4M3[codes.astype(np.intp)]


def _nearest_code(v, mags, sign_bit, vmax):
    """Brute-force nearest finite code for each float32 in ``v``.

    ``mags[i]`` is the magnitude of code i (codes 0..len-1 are the
    non-negative finite ones, in increasing order); ``sign_bit`` is the code
    bit that holds the sign.
    """
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("NaN input to an encoder")
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    idx = np.arange(mags.size)
    even = (idx & 1) == 0
    for lo in range(0, flat.size, _CHUNK):
        part = flat[lo:lo + _CHUNK]
        a = np.minimum(np.abs(part.astype(np.float64)), vmax)
        dist = np.abs(a[:, None] - mags[None, :])
        best = dist == dist.min(axis=1, keepdims=True)
        best_even = best & even[None, :]
        pick = np.where(best_even.any(axis=1), best_even.argmax(axis=1),
                        best.argmax(axis=1))
        neg = np.signbit(part)
        out[lo:lo + _CHUNK] = (pick | (neg.astype(np.intp) << sign_bit)).astype(np.uint8)
    return out.reshape(v.shape)


def encode_e2m1(v):
    """float32 -> E2M1 code (uint8 0..15), nearest, ties to even, saturating."""
    return _nearest_code(v, _E2M1[:8], 3, E2M1_MAX)


def encode_e4m3(v):
    """float32 -> E4M3FN code (uint8), nearest, ties to even, saturating."""
    return _nearest_code(v, _E4M3[:127], 7, E4M3_MAX)
