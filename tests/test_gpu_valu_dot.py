"""GPU parity of the VALU packed-dot path (valu_dot = 1, the alternative the
MFMA is measured against), through the C ABI, against the float64 oracle.

Bar: |y_gpu - y_ref| <= 2e-3 * sum_k |x * w| + 1e-3 per element; exact for
one-hot activations (each product and the block-scale multiply are exact in
fp32, and a power-of-two tensor scale keeps them so)."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import assert_within_tolerance, gpu_quantize, oracle_quantize, oracle_y, say, to_dev, to_host
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu

# (n, k, split, waves, k_slices, depth): ragged N (37, 300, 1000 rows) and K
# (48, 272, 1552, 2304), one-unit ranges, K slices and split-K.
SHAPES = [(512, 1024, 0, 0, 0, 0), (37, 48, 1, 4, 1, 2), (300, 5120, 2, 8, 2, 3), (1000, 2304, 3, 4, 1, 4),
          (96, 1552, 1, 8, 4, 2), (33, 272, 1, 8, 8, 3), (16, 4096, 4, 4, 2, 2)]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "n{}-k{}-s{}-w{}-ks{}-d{}".format(*s))
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_valu_dot_parity(fmt, m, shape):
    n, k, split, waves, ks, depth = shape
    say("valu dot", fmt, m, shape)
    seed = 3000 + n + k + m
    w = workloads.weights(n, k, seed)
    x = workloads.activations(m, k, seed + 1)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    y = to_host(qt.gemm(to_dev(x), pw, split_k=split, waves=waves, k_slices=ks, depth=depth, valu_dot=1))
    y_ref, b = oracle_y(fmt, x, oracle_quantize(fmt, w))
    assert_within_tolerance(y, y_ref, b, f"{fmt} valu_dot m={m} {shape}")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k,s_t", [(64, 512, 1.0), (20, 272, 0.25)])
def test_valu_dot_one_hot_is_exact(fmt, n, k, s_t):
    """x = e_k in each row reads back column k of the dequantized weight bit
    for bit: random codes and block scales, a power-of-two tensor (or row)
    scale."""
    say("valu dot one-hot", fmt, n, k, s_t)
    if fmt == "nvfp4":
        codes = workloads.random_nibble_bytes(n, k, 5)
        scales = workloads.random_block_scale_codes(n, k, 6)
        pw = qt.pack_nvfp4(to_dev(codes), to_dev(scales), s_t, n, k)
        wdq = oracle.dequantize_nvfp4(oracle.unpack_nibbles(codes), scales, s_t)
    else:
        codes = workloads.random_fp8_codes(n, k, 7)
        rs = np.full(n, s_t, np.float32)
        pw = qt.pack_fp8(to_dev(codes), to_dev(rs), n, k)
        wdq = oracle.dequantize_fp8(codes, rs)
    ks = [0, 1, 7, 8, 15, 16, 31, 63, 64, 255, k - 1, k - 2]
    for c0 in range(0, len(ks), 4):
        chunk = ks[c0:c0 + 4]
        x = np.zeros((len(chunk), k), np.float16)
        for i, kk in enumerate(chunk):
            x[i, kk] = 1.0
        y = to_host(qt.gemm(to_dev(x), pw, valu_dot=1))
        for i, kk in enumerate(chunk):
            assert np.all(np.abs(wdq[:, kk]) < 65504)
            assert np.array_equal(y[i].astype(np.float64), wdq[:, kk]), (fmt, kk)


@pytest.mark.parametrize("fmt,name,m", [("nvfp4", "gate_up", 1), ("nvfp4", "down", 1), ("nvfp4", "down", 4),
                                        ("fp8", "qkv", 2)])
def test_valu_dot_full_size_sampled(fmt, name, m):
    """27B shapes: the oracle recomputes a sample of output columns."""
    n, k = workloads.SHAPES[name]
    say("valu dot full size", fmt, name, m)
    w = workloads.weights(n, k, 71)
    x = workloads.activations(m, k, 72)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    y = to_host(qt.gemm(to_dev(x), pw, valu_dot=1))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                     np.random.default_rng(n + m).integers(0, n, 96)]))
    if fmt == "nvfp4":
        parts = oracle.quantize_nvfp4(w[cols], tensor_scale=oracle.nvfp4_tensor_scale(np.abs(w).max()))
    else:
        parts = oracle.quantize_fp8(w[cols])
    y_ref, b = oracle_y(fmt, x, parts)
    assert_within_tolerance(y[:, cols], y_ref, b, f"{fmt} {name} m={m} valu_dot")
    assert np.isfinite(y).all()
