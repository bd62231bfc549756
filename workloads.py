"""Seeded synthetic inputs for the skinny-GEMM workloads (shared by tests and bench).

This module holds input shapes and random-number recipes only: no
quantization, decoding or GEMM arithmetic. Both the CPU oracle and the HIP
path take their inputs from here, so the two sides see identical bytes.

The pages measure the kernels at the per-GPU shapes of a ~27B dense decoder
served under 4-way tensor parallelism ([P3] "What I actually built", the
bandwidth table: https://reddlx.com/feed/productivity-ai-news, post "Four
Tesla V100s from 2017 matched my RTX 5090 on single-request Qwen 3.8
decode"), without printing the shapes. The workloads below use the whole
(unsharded) matrices of such a decoder, hidden size 5120, on one GPU, plus a
small GEMV case that the oracle finishes in well under a second.

Recipes:
  W = 0.02 * standard_normal(float32)       (rng seeded per matrix)
  x = standard_normal(float32) -> float16    (all M rows independent)
  seed = crc32("<workload>/<matrix>/<W|x>")
"""

import zlib

import numpy as np

# (N, K) of each matrix: N output features, K reduction length.
SHAPES = {
    "gemv": (512, 1024),
    "gate_up": (34816, 5120),
    "down": (5120, 17408),
    "qkv": (7168, 5120),
    "o_proj": (5120, 5120),
    "lm_head": (151936, 5120),
    # one GPU's share of each matrix under 4-way tensor parallelism: the
    # column-parallel ones (qkv, gate_up) cut along N, the row-parallel ones
    # (o_proj, down) along K
    "qkv_tp4": (1792, 5120),
    "o_proj_tp4": (5120, 1280),
    "gate_up_tp4": (8704, 5120),
    "down_tp4": (5120, 4352),
}

# Workloads by name: (format, M values, matrices).
WORKLOADS = {
    "nvfp4_gemv_m1": ("nvfp4", (1,), ("gemv",)),
    "nvfp4_27b_m1": ("nvfp4", (1,), ("gate_up", "down")),
    "nvfp4_27b_m8": ("nvfp4", (8,), ("gate_up", "down", "qkv", "o_proj")),
    "fp8_27b_m124": ("fp8", (1, 2, 4), ("qkv", "down")),
    # 64 layers of [qkv FP8, o_proj FP8, gate_up NVFP4, down NVFP4] + NVFP4 lm_head
    "decode_step_27b": ("mixed", (1, 2, 4, 8), ("qkv", "o_proj", "gate_up", "down", "lm_head")),
    # per-rank shapes of 4-way tensor parallelism, and the 16-row verify block
    "nvfp4_27b_tp4": ("nvfp4", (1, 8), ("qkv_tp4", "o_proj_tp4", "gate_up_tp4", "down_tp4")),
    "nvfp4_27b_m16": ("nvfp4", (16,), ("gate_up", "down")),
}

DECODE_LAYERS = 64
DECODE_LAYER_MATS = (("qkv", "fp8"), ("o_proj", "fp8"), ("gate_up", "nvfp4"), ("down", "nvfp4"))

W_STD = 0.02


def seed_for(workload, matrix, kind):
    return zlib.crc32(f"{workload}/{matrix}/{kind}".encode())


def weights(n, k, seed, rows=None):
    """float32 W[N, K] = 0.02 * N(0, 1).

    ``rows`` (a slice) returns only those rows, bit-identical to the same rows
    of the full matrix (the generator draws row by row in blocks).
    """
    rng = np.random.default_rng(seed)
    if rows is None:
        return (np.float32(W_STD) * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    start, stop, _ = rows.indices(n)
    # Skip whole rows by drawing and discarding in bounded chunks.
    chunk = max(1, (1 << 24) // max(k, 1))
    r = 0
    while r + chunk <= start:
        rng.standard_normal((chunk, k), dtype=np.float32)
        r += chunk
    if start > r:
        rng.standard_normal((start - r, k), dtype=np.float32)
    out = rng.standard_normal((stop - start, k), dtype=np.float32)
    return (np.float32(W_STD) * out).astype(np.float32)


def activations(m, k, seed):
    """float16 x[M, K] from N(0, 1) float32 samples (round to nearest even)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


def random_nibble_bytes(n, k, seed):
    """Uniform random canonical NVFP4 code bytes [N, K/2] (every byte valid)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)


def random_block_scale_codes(n, k, seed, lo=0x00, hi=0x7E):
    """Random non-negative finite E4M3 scale codes [N, K/16] in [lo, hi]."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(n, k // 16), dtype=np.uint8)


def random_fp8_codes(n, k, seed):
    """Random E4M3 codes [N, K] avoiding the two NaN codes 0x7F and 0xFF."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)
