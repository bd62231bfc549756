"""Pins for oracle.quantize and oracle.layout: hand-computed cases, an
independent library encoder (torch float8_e4m3fn) for every scale and FP8
code, and invariants of the recipe."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from golden_io import load_case


def _torch_e4m3_codes(v):
    v = np.clip(np.asarray(v, np.float32), -448, 448)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_nvfp4_hand_case():
    case = load_case("nvfp4_hand_case.json")
    codes, sc, s_t = oracle.quantize_nvfp4(case["W"])
    assert s_t == np.float32(case["tensor_scale"])
    assert np.array_equal(sc, case["block_scale_codes"])
    assert np.array_equal(codes, case["codes"])
    assert np.array_equal(oracle.pack_nibbles(codes), case["packed_codes"])
    wdq = oracle.dequantize_nvfp4(codes, sc, s_t)
    assert np.array_equal(wdq, case["dequantized"])
    assert np.array_equal(np.signbit(wdq), np.signbit(case["dequantized"]))


def test_fp8_hand_case():
    case = load_case("fp8_hand_case.json")
    codes, rs = oracle.quantize_fp8(case["W"])
    assert np.array_equal(rs, case["row_scales"])
    assert np.array_equal(codes, case["codes"])


def test_pack_unpack_round_trip_and_nibble_order():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, (5, 64), dtype=np.uint8)
    p = oracle.pack_nibbles(c)
    assert p.shape == (5, 32)
    assert np.array_equal(oracle.unpack_nibbles(p), c)
    assert p[0, 0] == (c[0, 0] | (c[0, 1] << 4))


def _w(n=64, k=256, seed=11):
    return workloads.weights(n, k, seed)


def test_nvfp4_block_scales_match_torch_encoder():
    w = _w()
    codes, sc, s_t = oracle.quantize_nvfp4(w)
    amax_b = np.abs(w.reshape(w.shape[0], -1, 16)).max(axis=2)
    ratio = (amax_b / np.float32(6)) / np.float32(s_t)
    assert np.array_equal(sc, _torch_e4m3_codes(ratio))
    assert s_t == np.float32(np.abs(w).max()) / np.float32(2688)


def test_nvfp4_amax_element_encodes_to_six_with_top_scale():
    w = _w()
    codes, sc, s_t = oracle.quantize_nvfp4(w)
    n, k = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert sc[n, k // 16] == 0x7E
    assert codes[n, k] == (0x7 if w[n, k] > 0 else 0xF)


def test_nvfp4_codes_are_nearest_and_requantize_to_themselves():
    w = _w(32, 512, 5)
    codes, sc, s_t = oracle.quantize_nvfp4(w)
    d = (oracle.decode_e4m3(sc).astype(np.float32) * s_t).astype(np.float32)
    q = (w.reshape(32, -1, 16) / d[:, :, None]).reshape(32, 512).astype(np.float64)
    vals = oracle.decode_e2m1(codes)
    # nearest: no E2M1 value is closer to min(|w/d|, 6) than the chosen one
    allv = oracle.e2m1_table()[:8]
    a = np.minimum(np.abs(q), 6.0)
    best = np.min(np.abs(a[..., None] - allv), axis=-1)
    assert np.all(np.abs(a - np.abs(vals)) == best)
    # re-quantizing the dequantized weights with the same scales is a fixed point
    wdq = oracle.dequantize_nvfp4(codes, sc, s_t).astype(np.float32)
    codes2, sc2, _ = oracle.quantize_nvfp4(wdq, tensor_scale=s_t)
    # a block whose largest code is below 6 may get a smaller scale the second
    # time; where the scale is unchanged the codes must be too
    same = np.repeat(sc2 == sc, 16, axis=1)
    assert same.mean() > 0.5
    assert np.array_equal(codes2[same], codes[same])


def test_nvfp4_error_bound_random():
    w = _w(16, 1024, 9)
    codes, sc, s_t = oracle.quantize_nvfp4(w)
    wdq = oracle.dequantize_nvfp4(codes, sc, s_t)
    d = np.repeat(oracle.decode_e4m3(sc) * np.float64(s_t), 16, axis=1)
    # half an E2M1 gap at the chosen magnitude is at most 1 (gap 2 between 4 and 6),
    # and the scale was rounded from amax_b/6 so |w|/d <= 6 * (1 + 1/16) before saturation
    assert np.all(np.abs(w - wdq) <= 1.0 * d + 1e-30)


def test_nvfp4_zero_tensor_and_zero_block():
    w = np.zeros((2, 32), np.float32)
    w[1, 16] = -0.0
    codes, sc, s_t = oracle.quantize_nvfp4(w)
    assert s_t == 1.0 and not sc.any()
    assert codes[1, 16] == 0x8 and codes[0].sum() == 0


def test_fp8_codes_match_torch_encoder_and_amax_is_448():
    w = _w(48, 320, 21)
    w[3] = 0.0
    codes, rs = oracle.quantize_fp8(w)
    assert rs[3] == 1.0 and not codes[3].any()
    live = np.arange(48) != 3
    assert np.array_equal(rs[live], (np.abs(w[live]).max(axis=1) / np.float32(448)).astype(np.float32))
    assert np.array_equal(codes, _torch_e4m3_codes(w / rs[:, None]))
    j = np.argmax(np.abs(w[live]), axis=1)
    top = codes[live][np.arange(47), j]
    assert np.all((top & 0x7F) == 0x7E)


def test_quantizers_reject_non_finite_and_bad_k():
    w = np.ones((2, 32), np.float32)
    w[0, 0] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_nvfp4(w)
    with pytest.raises(ValueError):
        oracle.quantize_fp8(w)
    with pytest.raises(ValueError):
        oracle.quantize_nvfp4(np.ones((2, 24), np.float32))


def test_workload_row_slices_match_full_matrix():
    full = workloads.weights(300, 96, 77)
    part = workloads.weights(300, 96, 77, rows=slice(130, 171))
    assert np.array_equal(full[130:171], part)
