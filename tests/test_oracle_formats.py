"""Pins for oracle.formats: tables and encoders checked against things other than
themselves (torch's float8_e4m3fn, the OCP E2M1 value table, hand-listed ties,
nearest-value invariants)."""

import numpy as np
import pytest
import torch

import oracle
from golden_io import load_table


def _torch_e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_table_matches_torch_all_256_codes():
    ours = oracle.e4m3_table()
    ref = _torch_e4m3_values()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0


def test_e2m1_table_matches_ocp_value_list():
    rows = load_table("e2m1_values.txt")
    tab = oracle.e2m1_table()
    assert len(rows) == 16
    for code_s, val_s in rows:
        code = int(code_s, 16)
        val = float(val_s)
        assert tab[code] == val, (code, tab[code], val)
        assert np.signbit(tab[code]) == np.signbit(val)


def test_e2m1_table_structure():
    tab = oracle.e2m1_table()
    pos = tab[:8]
    assert np.all(np.diff(pos) > 0)                      # magnitude grows with code
    assert np.array_equal(tab[8:], -pos)                 # sign bit is bit 3
    assert set(np.nonzero(tab == 0)[0]) == {0, 8}
    # every E2M1 value is an E4M3 value (the formats nest), so decoding through
    # torch's E4M3 after an E4M3 encode must give back the same number
    t = torch.tensor(tab, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(t, tab)


def _e4m3_sweep():
    pos = np.sort(oracle.e4m3_table()[:127])
    mids = (pos[:-1] + pos[1:]) / 2
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)  # midpoints exact in fp32
    around = np.concatenate([mids32, np.nextafter(mids32, np.float32(0)), np.nextafter(mids32, np.float32(1e9)),
                             pos.astype(np.float32)])
    rng = np.random.default_rng(1234)
    logu = np.exp(rng.uniform(np.log(1e-6), np.log(460.0), 200000)).astype(np.float32)
    lin = rng.uniform(0, 1.0 / 64, 50000).astype(np.float32)  # subnormal band
    v = np.concatenate([around, logu, lin, [0.0]]).astype(np.float32)
    return np.concatenate([v, -v]).astype(np.float32)


def test_encode_e4m3_matches_torch_round_to_nearest_even():
    v = _e4m3_sweep()
    ours = oracle.encode_e4m3(v)
    # torch's fp32 -> float8_e4m3fn rounds to nearest even but gives NaN above
    # 464; clamp to the finite range first (our encoder saturates).
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch maps -0.0 inputs and tiny negatives to 0x80 as well
    assert np.array_equal(ours, ref)


def test_encode_e4m3_saturates_and_keeps_sign():
    v = np.array([448, 449, 464, 465, 480, 1e30, -1e30, np.inf, -np.inf, -0.0, -1e-12], np.float32)
    assert list(oracle.encode_e4m3(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x80, 0x80]


def test_encode_e4m3_idempotent_on_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.decode_e4m3(codes).astype(np.float32)
    assert np.array_equal(oracle.encode_e4m3(vals), codes)


def test_encode_e2m1_ties_and_saturation_fixture():
    rows = load_table("e2m1_rounding.txt")
    v = np.array([float(a) for a, _ in rows], np.float32)
    want = np.array([int(b, 16) for _, b in rows], np.uint8)
    assert np.array_equal(oracle.encode_e2m1(v), want)


def test_encode_e2m1_is_nearest_on_dense_sweep():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-7, 7, 100000), np.linspace(-6.5, 6.5, 26001)]).astype(np.float32)
    c = oracle.encode_e2m1(v)
    got = oracle.decode_e2m1(c)
    allv = oracle.e2m1_table()[:8]
    clipped = np.clip(v.astype(np.float64), -6, 6)
    best = np.min(np.abs(np.abs(clipped)[:, None] - allv[None, :]), axis=1)
    assert np.all(np.abs(np.abs(clipped) - np.abs(got)) == best)
    nz = got != 0
    assert np.all(np.sign(got[nz]) == np.sign(v[nz]))


def test_encode_e2m1_idempotent():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(oracle.encode_e2m1(oracle.decode_e2m1(codes).astype(np.float32)), codes)


def test_encoders_reject_nan():
    with pytest.raises(ValueError):
        oracle.encode_e2m1(np.array([1.0, np.nan], np.float32))
    with pytest.raises(ValueError):
        oracle.encode_e4m3(np.array([np.nan], np.float32))


def test_decode_rejects_out_of_range_e2m1():
    with pytest.raises(ValueError):
        oracle.decode_e2m1(np.array([16], np.uint8))
