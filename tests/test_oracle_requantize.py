"""Pins for oracle.requantize (FP8 -> NVFP4): the fp32 dequantize against
torch's float8_e4m3fn decode and fp32 multiply, a hand-worked block, a
lossless case (FP8 values already on the NVFP4 grid) and the NVFP4 error
bound on random FP8 weights."""

import numpy as np
import torch

import oracle
import workloads


def test_fp8_dequantize_f32_matches_torch():
    codes = workloads.random_fp8_codes(64, 256, 1)
    rs = (np.random.default_rng(2).random(64).astype(np.float32) + 0.01) * 0.01
    rs[3] = 1.0
    rs[5] = np.float32(2.0 ** -20)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(rs)[:, None]
    got = oracle.dequantize_fp8_f32(codes, rs)
    assert got.dtype == np.float32
    assert np.array_equal(got.view(np.uint32), ref.numpy().view(np.uint32))


def test_requantize_hand_block():
    # one row of 16 FP8 codes, row scale 0.5:
    #   0x38 = 1.0, 0x40 = 2.0, 0x44 = 3.0, 0x48 = 4.0, 0x30 = 0.5, 0x00 = 0, 0xB8 = -1.0, 0x3C = 1.5
    codes = np.array([[0x38, 0x40, 0x44, 0x48, 0x30, 0x00, 0xB8, 0x3C] * 2], np.uint8)
    rs = np.array([0.5], np.float32)
    w = oracle.dequantize_fp8_f32(codes, rs)
    assert w[0, :8].tolist() == [0.5, 1.0, 1.5, 2.0, 0.25, 0.0, -0.5, 0.75]
    c, sc, s_t = oracle.requantize_fp8_to_nvfp4(codes, rs)
    # amax 2.0: s_t = 2/2688; the block scale (2/6)/s_t = 448 -> E4M3 0x7E; d = fl(448 * s_t)
    # = fl(1/3), and w/d in fp32 is 3 * w: 1.5, 3, 4.5 -> 4, 6, 0.75 -> 1 (a tie: to the even
    # code), 0, -1.5, 2.25 -> 2
    d = np.float32(np.float32(448.0) * np.float32(np.float32(2.0) / np.float32(2688.0)))
    assert d == np.float32(1.0) / np.float32(3.0) and np.float32(0.25) / d == np.float32(0.75)
    assert s_t == np.float32(np.float32(2.0) / np.float32(2688.0))
    assert sc.tolist() == [[0x7E]]
    assert c[0, :8].tolist() == [0x3, 0x5, 0x6, 0x7, 0x2, 0x0, 0xB, 0x4]
    assert np.array_equal(c[0, 8:], c[0, :8])


def test_requantize_lossless_when_fp8_values_sit_on_the_nvfp4_grid():
    # every 16-block holds E2M1 magnitudes times 1/2 and reaches 3 = 6/2, so
    # every block scale is 448 and every E2M1 code is 2 * value exactly
    rng = np.random.default_rng(4)
    grid = np.array([0x00, 0x28, 0x30, 0x34, 0x38, 0x3C, 0x40, 0x44], np.uint8)  # 0 .25 .5 .75 1 1.5 2 3
    n, k = 8, 256
    codes = grid[rng.integers(0, 8, (n, k))]
    codes[:, ::16] = 0x44
    codes |= (rng.random((n, k)) < 0.5).astype(np.uint8) << 7
    rs = np.ones(n, np.float32)
    c, sc, s_t = oracle.requantize_fp8_to_nvfp4(codes, rs)
    assert (sc == 0x7E).all()
    want = oracle.dequantize_fp8_f32(codes, rs).astype(np.float64) * 2
    assert np.array_equal(oracle.decode_e2m1(c), want)


def test_requantize_error_bound_on_random_weights():
    codes = workloads.random_fp8_codes(32, 512, 7)
    rs = np.random.default_rng(8).random(32).astype(np.float32) * 1e-2 + 1e-4
    w = oracle.dequantize_fp8_f32(codes, rs).astype(np.float64)
    c, sc, s_t = oracle.requantize_fp8_to_nvfp4(codes, rs)
    wq = oracle.dequantize_nvfp4(c, sc, s_t)
    d = np.repeat(oracle.decode_e4m3(sc), 16, axis=1) * np.float64(s_t)
    # within one E2M1 step of the block's scale (half the widest gap, 4 -> 6,
    # is one d), and exact where the value is 0
    assert np.all(np.abs(wq - w) <= d * 1.0 + 1e-30)
    assert np.all(wq[w == 0] == 0)
    # the conversion costs accuracy: report that it is lossy but bounded
    rel = np.sqrt(np.mean((wq - w) ** 2) / np.mean(w ** 2))
    assert 0.01 < rel < 0.2
