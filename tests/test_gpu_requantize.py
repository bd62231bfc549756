"""GPU parity of the offline FP8 -> NVFP4 conversion (through the C ABI):
bit-exact codes, block scales and tensor scale against the oracle, and the
converted weight multiplies like the oracle's."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, assert_within_tolerance, gpu_quantize, say, to_dev, to_host
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu

SHAPES = [(64, 256), (37, 48), (1, 16), (130, 4112), (512, 1024)]


def _random_fp8(n, k, seed):
    codes = workloads.random_fp8_codes(n, k, seed)
    rs = (np.random.default_rng(seed + 1).random(n).astype(np.float32) * 3 + 0.05) * np.float32(2.0 ** -7)
    return codes, rs


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("source", ["random_codes", "quantized_weights"])
def test_requantize_matches_oracle(n, k, source):
    say("requantize", n, k, source)
    if source == "random_codes":
        codes, rs = _random_fp8(n, k, n + k)
        c8, r8 = to_dev(codes), to_dev(rs)
    else:
        pw, (c8, r8) = gpu_quantize("fp8", to_dev(workloads.weights(n, k, n * 3 + k)))
        codes, rs = to_host(c8), to_host(r8)
    c4, sc, s_t = qt.requantize_fp8_to_nvfp4(c8, r8)
    rc, rsc, rst = oracle.requantize_fp8_to_nvfp4(codes, rs)
    assert np.float32(s_t) == rst
    assert np.array_equal(to_host(sc), rsc)
    assert np.array_equal(to_host(c4), oracle.pack_nibbles(rc))


def test_requantized_weight_multiplies_like_the_oracle():
    say("requantize then gemm")
    n, k, m = 300, 2304, 8
    w = workloads.weights(n, k, 61)
    pw8, (c8, r8) = gpu_quantize("fp8", to_dev(w))
    c4, sc, s_t = qt.requantize_fp8_to_nvfp4(c8, r8)
    pw4 = qt.pack_nvfp4(c4, sc, s_t, n, k)
    x = workloads.activations(m, k, 62)
    y = to_host(qt.gemm(to_dev(x), pw4))
    rc, rsc, rst = oracle.requantize_fp8_to_nvfp4(to_host(c8), to_host(r8))
    y_ref, b = oracle.gemm_nvfp4(x, rc, rsc, rst)
    assert_within_tolerance(y, y_ref, b, "requantized gemm")
    # the FP8 original and its NVFP4 conversion differ by the conversion's
    # rounding, not by the GEMM: the NVFP4 result is closer to its own oracle
    y8 = to_host(qt.gemm(to_dev(x), pw8)).astype(np.float64)
    assert np.abs(y.astype(np.float64) - y_ref).mean() < np.abs(y8 - y_ref).mean()


def test_requantize_full_size_qkv_sampled_rows():
    """The 27B qkv (7168 x 5120) in FP8, converted on the GPU; the oracle
    converts a sample of rows with the tensor scale of the whole matrix."""
    n, k = workloads.SHAPES["qkv"]
    say("requantize full qkv")
    w = workloads.weights(n, k, workloads.seed_for("fp8_27b_m124", "qkv", "W"))
    pw8, (c8, r8) = gpu_quantize("fp8", to_dev(w))
    c4, sc, s_t = qt.requantize_fp8_to_nvfp4(c8, r8)
    codes, rs = to_host(c8), to_host(r8)
    amax = np.abs(oracle.dequantize_fp8_f32(codes, rs)).max()
    assert np.float32(s_t) == oracle.nvfp4_tensor_scale(amax)
    rows = np.unique(np.concatenate([[0, 1, n - 1], np.random.default_rng(5).integers(0, n, 40)]))
    wsub = oracle.dequantize_fp8_f32(codes[rows], rs[rows])
    rc, rsc, rst = oracle.quantize_nvfp4(wsub, tensor_scale=oracle.nvfp4_tensor_scale(amax))
    sel = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(to_host(sc.index_select(0, sel)), rsc)
    assert np.array_equal(to_host(c4.index_select(0, sel)), oracle.pack_nibbles(rc))
