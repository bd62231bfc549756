"""GPU parity of the greedy-argmax epilogue (through the C ABI): each row's
index must be one the oracle admits as the argmax under the GEMM bound
(oracle.argmax_candidates; exact whenever the top logit is clear of the
others by more than the bound), its value must be that logit to within the
bound, equal logits must give the smallest index, and the workspace counters
must be back at zero after every call."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, gpu_quantize, oracle_quantize, oracle_y, say, to_dev, to_host
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu

CONTROL = 64 * 16 * 8  # the workspace's control block: 64 x 16 argmax key slots


def _check(idx, val, y_ref, b, what):
    cand = oracle.argmax_candidates(y_ref, b)
    tol = oracle.tolerance(b)
    rows = np.arange(y_ref.shape[0])
    assert ((idx >= 0) & (idx < y_ref.shape[1])).all(), what
    assert cand[rows, idx].all(), f"{what}: index outside the admissible set"
    assert (np.abs(val.astype(np.float64) - y_ref[rows, idx]) <= tol[rows, idx]).all(), f"{what}: value"
    # where the oracle's winner is clear of the rest by more than the bound, it is unique
    unique = cand.sum(axis=1) == 1
    assert (idx[unique] == y_ref[unique].argmax(axis=1)).all(), what


def _parity(fmt, m, n, k, seed, **kw):
    w = workloads.weights(n, k, seed)
    x = workloads.activations(m, k, seed + 1)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    idx, val = qt.gemm_argmax(to_dev(x), pw, **kw)
    y_ref, b = oracle_y(fmt, x, oracle_quantize(fmt, w))
    _check(to_host(idx), to_host(val), y_ref, b, f"{fmt} m={m} n={n} k={k} {kw}")


SHAPES = [(512, 1024), (1000, 2304), (96, 5120), (33, 256)]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 3, 8, 16])
def test_argmax_parity(fmt, m, n, k):
    say("argmax", fmt, m, n, k)
    _parity(fmt, m, n, k, seed=5000 + n + k + m)


LAUNCHES = [dict(split_k=2, waves=8, depth=2, k_slices=2), dict(split_k=3, waves=4, depth=3, k_slices=1),
            dict(split_k=1, waves=8, depth=3, k_slices=4), dict(split_k=6, waves=8, depth=2, k_slices=1),
            dict(split_k=1, waves=4, depth=2, k_slices=1),
            # the ring activation stage (x_stage 2)
            dict(split_k=1, waves=8, depth=2, k_slices=1, x_stage=2), dict(split_k=2, waves=8, depth=3, k_slices=2, x_stage=2),
            dict(split_k=1, waves=4, depth=4, k_slices=2, x_stage=2),
            # leading groups whole, the others split
            dict(split_k=4, waves=8, depth=2, k_slices=1, x_stage=2, whole_groups=6),
            dict(split_k=2, waves=4, depth=3, k_slices=2, x_stage=1, whole_groups=17)]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("kw", LAUNCHES, ids=lambda d: "-".join(str(v) for v in d.values()))
def test_argmax_launch_shapes(fmt, kw):
    """In-workgroup logits and the split-K reduction's logits, ragged N."""
    say("argmax launch", fmt, kw)
    _parity(fmt, 5, 1000, 2304, seed=91, **kw)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_argmax_equal_logits_take_the_smallest_index(fmt):
    """Rows 100, 700 and 701 of W are the same large row aligned with x: their
    logits are equal bit for bit (same codes, same arithmetic) and the
    largest, so the answer is 100 in every activation row, every time."""
    say("argmax ties", fmt)
    n, k, m = 1024, 2048, 4
    rng = np.random.default_rng(8)
    x = workloads.activations(m, k, 9)
    x[1:] = x[0]
    w = workloads.weights(n, k, 10)
    top = (0.05 * np.sign(x[0].astype(np.float32))).astype(np.float32)
    for r in (100, 700, 701):
        w[r] = top
    w[rng.integers(0, n, 20)] *= 1.5
    pw, _ = gpu_quantize(fmt, to_dev(w))
    ws = qt.argmax_workspace(pw, m)
    for _ in range(3):
        idx, val = qt.gemm_argmax(to_dev(x), pw, workspace=ws)
        assert (to_host(idx) == 100).all()
        assert not to_host(ws[:256 + CONTROL]).any()   # 64 n-tile counters (256 B), control block
    y_ref, b = oracle_y(fmt, x, oracle_quantize(fmt, w))
    assert y_ref[0, 100] == y_ref[0].max()


def test_argmax_workspace_reuse_across_m_and_repeat():
    say("argmax reuse")
    n, k = 2000, 4096
    w = workloads.weights(n, k, 12)
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    ws = qt.argmax_workspace(pw, 16, split_k=4)
    ref = {}
    for m in (8, 3, 16, 8, 1, 3):
        x = to_dev(workloads.activations(m, k, 13 + m))
        idx, val = qt.gemm_argmax(x, pw, workspace=ws, split_k=4)
        got = (to_host(idx).tolist(), to_host(val).view(np.uint32).tolist())
        if m in ref:
            assert got == ref[m]
        ref[m] = got
        assert not to_host(ws[:512 + CONTROL]).any()   # 125 n-tile counters (512 B), control block


def _lm_head_oracle(x, codes, scales, s_t, chunk=8192):
    n = codes.shape[0]
    y = np.empty((x.shape[0], n))
    b = np.empty((x.shape[0], n))
    for r0 in range(0, n, chunk):
        wdq = oracle.dequantize_nvfp4(oracle.unpack_nibbles(codes[r0:r0 + chunk]), scales[r0:r0 + chunk], s_t)
        y[:, r0:r0 + chunk], b[:, r0:r0 + chunk] = oracle.skinny_gemm(x, wdq)
    return y, b


def test_argmax_full_size_lm_head():
    """The 151936 x 5120 NVFP4 head at M = 1 and 8 (the decoder's greedy
    verify step). Canonical codes are drawn on the host and packed on the
    GPU; the oracle dequantizes them itself and computes every logit."""
    n, k = workloads.SHAPES["lm_head"]
    say("argmax full lm_head")
    codes = workloads.random_nibble_bytes(n, k, 21)
    scales = workloads.random_block_scale_codes(n, k, 22, lo=0x30, hi=0x40)
    s_t = 0.0078125
    pw = qt.pack_nvfp4(to_dev(codes), to_dev(scales), s_t, n, k)
    x = workloads.activations(8, k, 23)
    y_ref, b = _lm_head_oracle(x, codes, scales, s_t)
    for m in (1, 8):
        idx, val = qt.gemm_argmax(to_dev(x[:m]), pw)
        _check(to_host(idx), to_host(val), y_ref[:m], b[:m], f"lm_head m={m}")
    del pw
    torch.cuda.empty_cache()
