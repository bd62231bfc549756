"""Pins for oracle.gemm: hand-computed outputs, an independent
dequantize-then-matmul route in torch float64, and closed-form identities."""

import numpy as np
import torch

import oracle
import workloads
from golden_io import load_case


def _e2m1_by_bits(codes):
    """E2M1 decode by bit arithmetic (independent of the oracle's table)."""
    c = torch.as_tensor(codes.astype(np.int64))
    s = torch.where((c & 8) != 0, -1.0, 1.0).to(torch.float64)
    e = ((c >> 1) & 3).to(torch.float64)
    m = (c & 1).to(torch.float64)
    mag = torch.where(e == 0, m * 0.5, torch.pow(2.0, e - 1) * (1 + m / 2))
    return s * mag


def _e4m3_by_torch(codes):
    return torch.as_tensor(codes).view(torch.float8_e4m3fn).to(torch.float64)


def test_nvfp4_hand_case_y():
    case = load_case("nvfp4_hand_case.json")
    codes, sc, s_t = oracle.quantize_nvfp4(case["W"])
    y, b = oracle.gemm_nvfp4(case["x"], codes, sc, s_t)
    assert np.array_equal(y, case["y"])
    assert b[1, 0] == 5721.875


def test_fp8_hand_case_y():
    case = load_case("fp8_hand_case.json")
    codes, rs = oracle.quantize_fp8(case["W"])
    y, _ = oracle.gemm_fp8(case["x"], codes, rs)
    assert np.array_equal(y, case["y"])


def test_nvfp4_matches_independent_torch_route():
    n, k, m = 40, 512, 5
    w = workloads.weights(n, k, 101)
    x = workloads.activations(m, k, 102)
    codes, sc, s_t = oracle.quantize_nvfp4(w)
    y, b = oracle.gemm_nvfp4(x, codes, sc, s_t)
    wt = _e2m1_by_bits(codes) * _e4m3_by_torch(sc).repeat_interleave(16, dim=1) * float(s_t)
    yt = torch.as_tensor(x.astype(np.float64)) @ wt.T
    assert np.all(np.abs(y - yt.numpy()) <= 1e-12 * b)
    assert np.all(b >= np.abs(y))


def test_fp8_matches_independent_torch_route():
    n, k, m = 24, 384, 3
    w = workloads.weights(n, k, 103)
    x = workloads.activations(m, k, 104)
    codes, rs = oracle.quantize_fp8(w)
    y, b = oracle.gemm_fp8(x, codes, rs)
    wt = _e4m3_by_torch(codes) * torch.as_tensor(rs.astype(np.float64))[:, None]
    yt = torch.as_tensor(x.astype(np.float64)) @ wt.T
    assert np.all(np.abs(y - yt.numpy()) <= 1e-12 * b)


def test_closed_forms():
    n, k, m = 16, 256, 4
    w = workloads.weights(n, k, 105)
    x = workloads.activations(m, k, 106)
    codes, sc, s_t = oracle.quantize_nvfp4(w)
    y, _ = oracle.gemm_nvfp4(x, codes, sc, s_t)
    y_neg, _ = oracle.gemm_nvfp4(-x, codes, sc, s_t)
    assert np.array_equal(y_neg, -y)
    y2, _ = oracle.gemm_nvfp4(x, codes, sc, np.float32(2 * s_t))
    assert np.array_equal(y2, 2 * y)
    perm = np.random.default_rng(0).permutation(n)
    yp, _ = oracle.gemm_nvfp4(x, codes[perm], sc[perm], s_t)
    assert np.array_equal(yp, y[:, perm])
    for r in range(m):
        yr, _ = oracle.gemm_nvfp4(x[r:r + 1], codes, sc, s_t)
        assert np.allclose(yr[0], y[r], rtol=0, atol=1e-12)


def test_one_hot_activation_reads_back_one_weight():
    n, k = 8, 64
    codes = workloads.random_nibble_bytes(n, k, 1)
    sc = workloads.random_block_scale_codes(n, k, 2)
    c = oracle.unpack_nibbles(codes)
    wdq = oracle.dequantize_nvfp4(c, sc, np.float32(0.25))
    for kk in (0, 15, 16, 63):
        x = np.zeros((1, k), np.float16)
        x[0, kk] = 1
        y, _ = oracle.skinny_gemm(x, wdq)
        assert np.array_equal(y[0], wdq[:, kk])
        # the same weight from first principles: nibble of byte kk//2, scale kk//16
        nib = (codes[:, kk // 2] >> (4 * (kk % 2))) & 0xF
        assert np.array_equal(y[0], _e2m1_by_bits(nib).numpy() * _e4m3_by_torch(sc[:, kk // 16]).numpy() * 0.25)


def test_tolerance_formula():
    assert oracle.tolerance(0.0) == 1e-3
    assert np.isclose(oracle.tolerance(10.0), 0.021)


def test_argmax_candidates_clear_winner_and_near_ties():
    # b = 0 gives the bound 1e-3 on every element
    y = np.array([[0.0, 5.0, 1.0, 4.9],        # clear winner: index 1 alone
                  [2.0, 2.0015, -1.0, 1.9996],  # within 2e-3 of the top: 0, 1 and 3
                  [-3.0, -3.0, -3.0, -3.0]])   # all equal: every index
    b = np.zeros_like(y)
    c = oracle.argmax_candidates(y, b)
    assert c[0].tolist() == [False, True, False, False]
    assert c[1].tolist() == [True, True, False, True]
    assert c[2].all()
    # the exact argmax always qualifies, and a wider bound only adds indices
    rng = np.random.default_rng(3)
    yy = rng.standard_normal((50, 300))
    bb = rng.random((50, 300))
    c1 = oracle.argmax_candidates(yy, bb)
    assert c1[np.arange(50), yy.argmax(1)].all()
    assert (oracle.argmax_candidates(yy, 3 * bb) >= c1).all()
    # brute force on a small case: i qualifies iff some choice of values within the
    # bounds makes i the largest
    y3 = rng.standard_normal((200, 5)) * 2e-3
    b3 = np.zeros_like(y3)
    c3 = oracle.argmax_candidates(y3, b3)
    t = 1e-3
    for r in range(200):
        for i in range(5):
            best_i = y3[r, i] + t
            others = np.delete(y3[r] - t, i)
            assert c3[r, i] == (best_i >= others.max())
