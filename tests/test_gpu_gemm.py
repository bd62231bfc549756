"""GPU parity of qpn_gemm (through the C ABI) against the float64 oracle.

Bar: |y_gpu - y_ref| <= 2e-3 * sum_k |x * w| + 1e-3 per element; exact where
the arithmetic is exact (one-hot activations, negation, repeat runs)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (DEV, assert_within_tolerance, gpu_quantize, oracle_quantize, oracle_y,
                         say, to_dev, to_host)
import quantized_weight_skinny_amd as q
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu

SMALL = [(512, 1024), (37, 48), (100, 272), (16, 4096), (33, 2304), (300, 5120)]


def _parity(fmt, m, n, k, seed, **kw):
    w = workloads.weights(n, k, seed)
    x = workloads.activations(m, k, seed + 1)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    y = to_host(qt.gemm(to_dev(x), pw, **kw))
    parts = oracle_quantize(fmt, w)
    y_ref, b = oracle_y(fmt, x, parts)
    assert_within_tolerance(y, y_ref, b, f"{fmt} m={m} n={n} k={k} {kw}")
    return y


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k", SMALL)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 16])
def test_gemm_parity_small(fmt, m, n, k):
    say("gemm", fmt, m, n, k)
    _parity(fmt, m, n, k, seed=1000 + n + k + m)


LAUNCHES = [(1, 4, 2, 1), (2, 4, 3, 1), (3, 8, 4, 1), (5, 4, 6, 1), (7, 8, 8, 1), (0, 8, 0, 0),
            (4, 4, 8, 1), (1, 8, 6, 1), (1, 4, 3, 4), (1, 8, 3, 8), (2, 8, 4, 2), (3, 4, 2, 2),
            (1, 8, 2, 4), (7, 8, 3, 8)]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("split,waves,depth,k_slices", LAUNCHES)
def test_gemm_launch_shapes_agree(fmt, split, waves, depth, k_slices):
    n, k, m = 96, 1792, 5
    say("gemm tuned", fmt, split, waves, depth, k_slices)
    _parity(fmt, m, n, k, seed=77, split_k=split, waves=waves, depth=depth, k_slices=k_slices)


RING = qt.QPN_X_STAGE_RING
FULL_STAGE = qt.QPN_X_STAGE_FULL
# ring launches for m = 5: k_slices * m <= 4 * waves, depth 2..4
RING_LAUNCHES = [(1, 4, 2, 1), (1, 4, 3, 2), (1, 8, 4, 4), (2, 8, 2, 2), (3, 4, 4, 1), (7, 8, 3, 1),
                 (0, 8, 0, 0), (0, 0, 0, 0)]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("split,waves,depth,k_slices", RING_LAUNCHES)
def test_ring_stage_launch_shapes(fmt, split, waves, depth, k_slices):
    n, k, m = 96, 1792, 5
    say("gemm ring", fmt, split, waves, depth, k_slices)
    _parity(fmt, m, n, k, seed=77, split_k=split, waves=waves, depth=depth, k_slices=k_slices, x_stage=RING)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k", SMALL)
@pytest.mark.parametrize("m", [1, 3, 8, 16])
def test_ring_stage_parity_small(fmt, m, n, k):
    """The ring stage on ragged K tails (48, 272, 1552 ...), one-unit K ranges
    and every row count class."""
    say("gemm ring small", fmt, m, n, k)
    _parity(fmt, m, n, k, seed=2000 + n + k + m, x_stage=RING)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("m,n,k,split,waves,k_slices,depth", [
    (1, 512, 2304, 1, 4, 4, 3), (3, 100, 272, 1, 8, 2, 2), (8, 300, 1280, 1, 8, 2, 4),
    (8, 1024, 5120, 3, 8, 2, 2), (16, 64, 2304, 1, 8, 2, 3), (16, 640, 4352, 2, 4, 1, 4),
    (5, 33, 1552, 2, 8, 4, 2)])
def test_ring_and_full_stage_give_the_same_bits(fmt, m, n, k, split, waves, k_slices, depth):
    """Both stages feed the same MFMA sequence in the same order: for one
    launch shape the outputs agree bit for bit (the full stage without block
    columns, which the ring does not have)."""
    say("ring vs full", fmt, m, n, k, split, waves, k_slices, depth)
    w = workloads.weights(n, k, 31 + m)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    x = to_dev(workloads.activations(m, k, 32 + m))
    kw = dict(split_k=split, waves=waves, k_slices=k_slices, depth=depth)
    y_full = to_host(qt.gemm(x, pw, x_stage=FULL_STAGE, block_columns=2, **kw))
    y_ring = to_host(qt.gemm(x, pw, x_stage=RING, **kw))
    assert np.array_equal(y_full.view(np.uint16), y_ring.view(np.uint16))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("m,n,k,split,whole,waves,k_slices,depth,stage", [
    (8, 1000, 2304, 4, 20, 4, 2, 2, 2),      # 32 groups: 20 whole, 12 split four ways (ragged N)
    (1, 1000, 2304, 3, 50, 4, 4, 3, 1),      # full stage holding all of K for the whole groups
    (5, 512, 1552, 2, 7, 8, 2, 3, 2),        # ragged K tail, 8 groups: 7 whole, 1 split
    (16, 640, 4352, 6, 9, 8, 2, 2, 2),       # 10 groups, one split six ways
    (3, 96, 1792, 5, 1, 4, 1, 4, 1)])        # 2 groups: one whole, one split five ways
def test_whole_groups_with_split_k(fmt, m, n, k, split, whole, waves, k_slices, depth, stage):
    """The leading groups take all of K, the rest split it: every output within
    the bound, and reuse of the workspace leaves the same bits."""
    say("whole groups", fmt, m, n, k, split, whole, waves, k_slices, depth, stage)
    kw = dict(split_k=split, whole_groups=whole, waves=waves, k_slices=k_slices, depth=depth, x_stage=stage)
    y = _parity(fmt, m, n, k, seed=500 + whole, **kw)
    # the whole groups' outputs are the unsplit GEMM's bits
    w = workloads.weights(n, k, 500 + whole)
    x = to_dev(workloads.activations(m, k, 501 + whole))
    pw, _ = gpu_quantize(fmt, to_dev(w))
    y1 = to_host(qt.gemm(x, pw, split_k=1, waves=waves, k_slices=k_slices, depth=depth, x_stage=stage))
    rows = whole * 16 * (waves // k_slices)
    assert np.array_equal(y[:, :rows].view(np.uint16), y1[:, :rows].view(np.uint16))
    ws = qt.new_workspace(pw, m, **kw)
    again = [to_host(qt.gemm(x, pw, workspace=ws, **kw)) for _ in range(2)]
    assert np.array_equal(again[0].view(np.uint16), y.view(np.uint16))
    assert np.array_equal(again[1].view(np.uint16), y.view(np.uint16))
    assert not to_host(ws[:(-(-n // 16)) * 4]).any()


@pytest.mark.parametrize("m,n,k,groups,depth,stage", [
    (1, 16 * 37 - 5, 304, 5, 2, 1),     # 37 n-tiles: 8, 8, 7, 7, 7; ragged N and K
    (9, 16 * 37 - 5, 304, 5, 3, 2),
    (16, 720, 1552, 5, 2, 2),           # 45 n-tiles, 9 each
    (3, 720, 1552, 45, 3, 1),           # one n-tile each
    (16, 1000, 5120, 7, 2, 2),          # 63 n-tiles, 9 each, 20 units of K
    (8, 2000, 272, 16, 3, 2),           # 125 n-tiles: 13 workgroups of 8, 3 of 7
    (2, 2000, 272, 125, 2, 1)])
def test_uneven_grid(m, n, k, groups, depth, stage):
    """The uneven-group grid (9 wavefronts, `groups` workgroups sharing the
    n-tiles): every output within the bound, and the bits of the launch with
    one K slice and no split at the same depth and stage (each n-tile is
    summed over all of K by one wavefront in both), for fp16 and fp32 y."""
    say("uneven grid", m, n, k, groups, depth, stage)
    kw = dict(split_k=1, waves=9, k_slices=1, depth=depth, x_stage=stage, whole_groups=groups)
    y = _parity("nvfp4", m, n, k, seed=900 + groups + m, **kw)
    w = workloads.weights(n, k, 900 + groups + m)
    x = to_dev(workloads.activations(m, k, 901 + groups + m))
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    ref = dict(split_k=1, waves=8, k_slices=1, depth=depth, x_stage=stage)
    y8 = to_host(qt.gemm(x, pw, **ref))
    assert np.array_equal(y.view(np.uint16), y8.view(np.uint16))
    f9 = to_host(qt.gemm_f32(x, pw, **kw))
    f8 = to_host(qt.gemm_f32(x, pw, **ref))
    assert np.array_equal(f9.view(np.uint32), f8.view(np.uint32))


def test_ring_stage_takes_a_k_range_the_full_stage_cannot():
    """down (17408) at 16 rows in one K range: 557 KB of activations per
    workgroup do not fit LDS, the 3-unit ring does."""
    n, k, m = 256, 17408, 16
    say("ring long k", n, k, m)
    _parity("nvfp4", m, n, k, seed=41, split_k=1, waves=8, k_slices=2, x_stage=RING)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("k_slices", [2, 4, 8])
def test_k_slices_ragged(fmt, k_slices):
    """K slices that do not divide the K range evenly (and slices left empty)."""
    say("k slices ragged", fmt, k_slices)
    _parity(fmt, 3, 50, 1552, seed=88, waves=8, k_slices=k_slices)       # 7 units, ragged tail
    _parity(fmt, 2, 33, 256, seed=89, waves=8, k_slices=k_slices)        # 1 unit: most slices empty


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_split_k_workspace_reuse_is_deterministic(fmt):
    """The split-K arrival counters are left at zero by every call, so one
    workspace serves many calls (and different row counts) with identical bits."""
    n, k = 5120, 17408 // 4
    say("split-k reuse", fmt)
    w = workloads.weights(n, k, 21)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    ws = qt.new_workspace(pw, 16, split_k=6)
    assert ws.numel() >= qt.workspace_bytes(pw, 8, split_k=6, k_slices=2)
    assert ws is not None
    outs = []
    for m in (8, 3, 8, 16, 8):
        x = to_dev(workloads.activations(m, k, 22)[:m])
        outs.append((m, to_host(qt.gemm(x, pw, workspace=ws, split_k=6))))
    assert not to_host(ws[:(n // 16) * 4]).any()  # counters back at zero
    ref8 = outs[0][1]
    for m, y in outs:
        if m == 8:
            assert np.array_equal(y.view(np.uint16), ref8.view(np.uint16))
    parts = oracle_quantize(fmt, w)
    y_ref, b = oracle_y(fmt, workloads.activations(16, k, 22), parts)
    assert_within_tolerance(outs[3][1], y_ref, b, f"{fmt} split 6 m=16")


def test_gemm_vs_hand_case():
    say("gemm hand case")
    from golden_io import load_case
    case = load_case("nvfp4_hand_case.json")
    codes, scales, s_t = qt.quantize_nvfp4(to_dev(case["W"]))
    pw = qt.pack_nvfp4(codes, scales, s_t, 2, 32)
    y = to_host(qt.gemm(to_dev(case["x"]), pw))
    # every partial sum of the hand case is exact in fp32, so the only rounding
    # is the final one to fp16 (nearest even)
    assert np.array_equal(y, case["y"].astype(np.float16))


def _one_hot_check(fmt, n, k, s_t=1.0):
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
    ks = [0, 1, 7, 8, 15, 16, 31, 63, 64, 255, k - 1]
    x = np.zeros((len(ks), k), np.float16)
    for i, kk in enumerate(ks):
        x[i, kk] = 1.0
    y = to_host(qt.gemm(to_dev(x), pw))
    for i, kk in enumerate(ks):
        want = wdq[:, kk]
        assert np.all(np.abs(want) < 65504)
        assert np.array_equal(y[i].astype(np.float64), want), (fmt, kk)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_one_hot_reads_back_every_weight_exactly(fmt):
    """x = e_k picks one weight column: decoding must be bit-exact."""
    say("one hot", fmt)
    _one_hot_check(fmt, 64, 512)
    _one_hot_check(fmt, 20, 272, s_t=0.25)


def test_fp8_one_hot_covers_all_codes():
    say("fp8 all codes")
    n, k = 16, 256
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F] * 17, np.uint8)[: n * k].reshape(n, k)
    rs = np.ones(n, np.float32)
    pw = qt.pack_fp8(to_dev(codes), to_dev(rs), n, k)
    wdq = oracle.dequantize_fp8(codes, rs)
    x = np.eye(k, dtype=np.float16)[:16]
    for start in range(0, k, 16):
        x = np.eye(k, dtype=np.float16)[start:start + 16]
        y = to_host(qt.gemm(to_dev(x), pw))
        assert np.array_equal(y.astype(np.float64), wdq[:, start:start + 16].T)


def test_negation_and_repeat_are_bit_exact():
    say("negation / determinism")
    n, k, m = 300, 5120, 8
    w = workloads.weights(n, k, 9)
    x = workloads.activations(m, k, 10)
    for fmt in ("nvfp4", "fp8"):
        pw, _ = gpu_quantize(fmt, to_dev(w))
        xd = to_dev(x)
        y1 = to_host(qt.gemm(xd, pw))
        y2 = to_host(qt.gemm(xd, pw))
        yn = to_host(qt.gemm(-xd, pw))
        assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
        assert np.array_equal(yn, -y1)


def test_scale_doubling_and_row_permutation_are_exact():
    """Closed forms of y = x W~^T on the device: doubling the NVFP4 tensor
    scale (or the FP8 row scales) doubles the fp32 output exactly, and
    permuting W's rows permutes y's columns bit for bit (an output's
    arithmetic does not depend on where its row sits)."""
    say("scale doubling / row permutation")
    n, k, m = 304, 2304, 5
    w = to_dev(workloads.weights(n, k, 31))
    x = to_dev(workloads.activations(m, k, 32))
    codes, scales, s_t = qt.quantize_nvfp4(w)
    c8, rs = qt.quantize_fp8(w)
    packs = {
        "nvfp4": lambda idx, f: qt.pack_nvfp4(codes[idx].contiguous(), scales[idx].contiguous(), f * s_t, n, k),
        "fp8": lambda idx, f: qt.pack_fp8(c8[idx].contiguous(), (f * rs[idx]).contiguous(), n, k),
    }
    ident = torch.arange(n, device=DEV)
    perm = np.random.default_rng(33).permutation(n)
    pt = torch.from_numpy(perm).to(DEV)
    for fmt, pack in packs.items():
        pw, pw2, pwp = pack(ident, 1.0), pack(ident, 2.0), pack(pt, 1.0)
        for kw in ({}, dict(split_k=3), dict(k_slices=4, waves=8)):
            y1 = to_host(qt.gemm_f32(x, pw, **kw))
            assert np.array_equal(to_host(qt.gemm_f32(x, pw2, **kw)), 2 * y1), (fmt, kw)
            y = to_host(qt.gemm(x, pw, **kw))
            yp = to_host(qt.gemm(x, pwp, **kw))
            assert np.array_equal(yp.view(np.uint16), y[:, perm].view(np.uint16)), (fmt, kw)


def test_rows_of_a_batch_match_single_row_calls():
    say("batch rows")
    n, k = 128, 1024
    w = workloads.weights(n, k, 12)
    x = workloads.activations(8, k, 13)
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    y8 = to_host(qt.gemm(to_dev(x), pw))
    for r in range(8):
        # same per-column arithmetic for any M when K is not split differently
        # (one row with block columns off: block columns sum in another order)
        y1 = to_host(qt.gemm(to_dev(x[r:r + 1]), pw, block_columns=2))
        assert np.array_equal(y8[r], y1[0])


def test_output_guard_bytes_untouched():
    say("guard bytes")
    n, k, m = 50, 512, 3
    w = workloads.weights(n, k, 14)
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    buf = torch.full((m * n + 64,), 12345.0, dtype=torch.float16, device=DEV)
    out = buf[:m * n].view(m, n)
    qt.gemm(to_dev(workloads.activations(m, k, 15)), pw, out=out)
    tail = to_host(buf[m * n:])
    assert np.all(tail == np.float16(12345.0))


def test_binding_refuses_sizes_the_kernels_would_overrun():
    """The torch binding checks every tensor a kernel reads or writes against
    the weight's shape before any launch."""
    say("binding size checks")
    n, k, m = 48, 512, 2
    w = workloads.weights(n, k, 16)
    pw, (codes, scales, _) = gpu_quantize("nvfp4", to_dev(w))
    x = to_dev(workloads.activations(m, k, 17))
    for bad_x in (x[:, :k - 16].contiguous(), x.reshape(-1), torch.zeros((m, k + 16), dtype=torch.float16,
                                                                            device=DEV)):
        for call in (qt.gemm, qt.gemm_f32, qt.gemm_argmax):
            with pytest.raises(ValueError):
                call(bad_x, pw)
    with pytest.raises(ValueError):
        qt.gemm_swiglu(x[:, :256].contiguous(), pw)
    with pytest.raises(ValueError):
        qt.gemm_argmax(x, pw, idx=torch.empty(m - 1, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        qt.pack_nvfp4(codes[: n - 1].contiguous(), scales, 1.0, n, k)
    with pytest.raises(ValueError):
        qt.pack_nvfp4(codes, scales[:, :-1].contiguous(), 1.0, n, k)
    c8, rs = qt.quantize_fp8(to_dev(w))
    with pytest.raises(ValueError):
        qt.pack_fp8(c8, rs[:-1].contiguous(), n, k)
    with pytest.raises(ValueError):
        qt.pack_fp8(c8[:, :-16].contiguous(), rs, n, k)
    with pytest.raises(ValueError):
        qt.requantize_fp8_to_nvfp4(c8, rs[:-1].contiguous())
    # the well-formed calls still run
    assert qt.gemm(x, pw).shape == (m, n)
    assert qt.pack_fp8(c8, rs, n, k).n == n


def test_empty_and_degenerate_shapes():
    say("degenerate shapes")
    # K = 0: the empty sum
    pw = qt.pack_nvfp4(torch.zeros((4, 0), dtype=torch.uint8, device=DEV),
                       torch.zeros((4, 0), dtype=torch.uint8, device=DEV), 1.0, 4, 0)
    x = torch.zeros((2, 0), dtype=torch.float16, device=DEV)
    y = torch.full((2, 4), 7.0, dtype=torch.float16, device=DEV)
    qt.gemm(x, pw, out=y)
    assert not to_host(y).any()
    # ... through the ring stage too (automatic from 5 rows, or forced)
    for m, kw in ((8, {}), (2, dict(x_stage=qt.QPN_X_STAGE_RING))):
        x = torch.zeros((m, 0), dtype=torch.float16, device=DEV)
        y = torch.full((m, 4), 7.0, dtype=torch.float16, device=DEV)
        qt.gemm(x, pw, out=y, **kw)
        assert not to_host(y).any()
    # M = 0 and N = 0 do nothing
    pw2, _ = gpu_quantize("nvfp4", to_dev(workloads.weights(16, 32, 1)))
    qt.gemm(torch.zeros((0, 32), dtype=torch.float16, device=DEV), pw2)
    # N = 1, K = 16: a single block
    _parity("nvfp4", 1, 1, 16, seed=3)
    _parity("fp8", 3, 1, 16, seed=4)
    _parity("nvfp4", 16, 1, 16, seed=5)          # ring stage, one 16-element block


# Every (format, matrix) the bench times, with every M the bench or the
# 64-layer decode step (1, 2, 4, 8) runs it at (and gate_up at 9 rows, the
# first that takes the uneven grid).
FULL_M = {
    ("nvfp4", "gate_up"): (1, 2, 4, 8, 9, 16), ("nvfp4", "down"): (1, 2, 4, 8, 16), ("nvfp4", "qkv"): (1, 8),
    ("nvfp4", "o_proj"): (1, 3, 8), ("nvfp4", "lm_head"): (1, 2, 4, 8), ("nvfp4", "gemv"): (1,),
    ("nvfp4", "qkv_tp4"): (1, 8), ("nvfp4", "o_proj_tp4"): (1, 8), ("nvfp4", "gate_up_tp4"): (1, 8),
    ("nvfp4", "down_tp4"): (1, 8), ("fp8", "qkv"): (1, 2, 4, 8), ("fp8", "down"): (1, 2, 4, 7, 8),
    ("fp8", "o_proj"): (1, 2, 4, 8),
}

U32 = 2.0 ** -24


def _random_codes(fmt, n, k, seed):
    """Seeded random canonical codes at weight-like magnitudes: uniform E2M1
    codes with E4M3 block scales in [2^-3, 2] and s_t = 2^-6 (|w| <= 0.19), or
    uniform non-NaN E4M3 codes with row scales 2^-11 .. 2^-13 (|w| <= 0.22)."""
    if fmt == "nvfp4":
        return (workloads.random_nibble_bytes(n, k, seed),
                workloads.random_block_scale_codes(n, k, seed + 1, lo=0x20, hi=0x40), np.float32(2.0 ** -6))
    rs = np.float32(2.0) ** -np.random.default_rng(seed + 2).integers(11, 14, n).astype(np.float32)
    return workloads.random_fp8_codes(n, k, seed), rs.astype(np.float32)


def _pack(fmt, parts, n, k):
    if fmt == "nvfp4":
        codes, scales, s_t = parts
        return qt.pack_nvfp4(to_dev(codes), to_dev(scales), float(s_t), n, k)
    codes, rs = parts
    return qt.pack_fp8(to_dev(codes), to_dev(rs), n, k)


def _oracle_rows(fmt, parts, x, r0, r1):
    if fmt == "nvfp4":
        codes, scales, s_t = parts
        return oracle.gemm_nvfp4(x, oracle.unpack_nibbles(codes[r0:r1]), scales[r0:r1], s_t)
    codes, rs = parts
    return oracle.gemm_fp8(x, codes[r0:r1], rs[r0:r1])


@pytest.mark.parametrize("fmt,matrix", list(FULL_M))
def test_full_size_all_outputs(fmt, matrix):
    """27B-shaped matrices in the launch configuration the bench times, every
    output column of every M against the oracle (in row chunks): the fp16
    output within the acceptance bound, the fp32 output (same launch, same
    accumulator) within the fp32 summation bound gamma(K + 64) * sum|w x|,
    and the fp16 output equal to the fp32 one rounded to fp16 up to double
    rounding at exact ties. The fp32 bound is far tighter than the
    acceptance bound: a dropped or mis-scaled 16-element block shows there.
    Both sides take the same seeded canonical codes (the oracle's quantizer
    is too slow for whole matrices; quantization of the full-size matrices is
    checked on sampled rows in test_gpu_quantize_pack.py)."""
    n, k = workloads.SHAPES[matrix]
    ms = FULL_M[(fmt, matrix)]
    say("full size", fmt, matrix, ms, n, k)
    seed = workloads.seed_for("full_size", matrix, fmt)
    parts = _random_codes(fmt, n, k, seed)
    pw = _pack(fmt, parts, n, k)
    xs = {m: workloads.activations(m, k, seed + 10 + m) for m in ms}
    out = {}
    for m in ms:
        xd = to_dev(xs[m])
        out[m] = (to_host(qt.gemm(xd, pw)), to_host(qt.gemm_f32(xd, pw)))
    del pw
    torch.cuda.empty_cache()
    xall = np.concatenate([xs[m] for m in ms])
    offs = np.cumsum([0] + [m for m in ms])
    bound_f = (k + 64) * U32 / (1 - (k + 64) * U32)
    for r0 in range(0, n, 8192):
        r1 = min(n, r0 + 8192)
        y_ref, b = _oracle_rows(fmt, parts, xall, r0, r1)
        for i, m in enumerate(ms):
            y16, y32 = out[m][0][:, r0:r1], out[m][1][:, r0:r1]
            yr, bb = y_ref[offs[i]:offs[i + 1]], b[offs[i]:offs[i + 1]]
            what = f"{fmt} {matrix} m={m} rows {r0}.."
            assert_within_tolerance(y16, yr, bb, what)
            err = np.abs(y32.astype(np.float64) - yr)
            assert np.all(err <= bound_f * bb), (what, int((err > bound_f * bb).sum()))
            h = y32.astype(np.float16)
            diff = h.view(np.uint16) != y16.view(np.uint16)
            if diff.any():
                a, c, v = h[diff], y16[diff], y32[diff].astype(np.float64)
                assert np.all((np.nextafter(a, c) == c) & ((a.astype(np.float64) + c.astype(np.float64)) / 2 == v))


# Quantized synthetic weights at full size (quantize -> pack -> GEMM on the
# device), sampled output columns recomputed by the oracle from its own
# quantization of those rows.
FULL_SAMPLED = [("nvfp4", "gate_up", 1), ("nvfp4", "down", 8), ("nvfp4", "o_proj", 8), ("fp8", "qkv", 4),
                ("fp8", "down", 1), ("nvfp4", "lm_head", 2)]


@pytest.mark.parametrize("fmt,matrix,m", FULL_SAMPLED)
def test_full_size_quantized_sampled(fmt, matrix, m):
    n, k = workloads.SHAPES[matrix]
    say("full size quantized", fmt, matrix, m, n, k)
    wl = "decode_step_27b"
    w = workloads.weights(n, k, workloads.seed_for(wl, matrix, "W"))
    x = workloads.activations(m, k, workloads.seed_for(wl, matrix, "x"))
    wd = to_dev(w)
    pw, _ = gpu_quantize(fmt, wd)
    del wd
    y = to_host(qt.gemm(to_dev(x), pw))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                     np.random.default_rng(n + m).integers(0, n, 96)]))
    if fmt == "nvfp4":
        parts = oracle.quantize_nvfp4(w[cols], tensor_scale=oracle.nvfp4_tensor_scale(np.abs(w).max()))
    else:
        parts = oracle.quantize_fp8(w[cols])
    y_ref, b = oracle_y(fmt, x, parts)
    assert_within_tolerance(y[:, cols], y_ref, b, f"{fmt} {matrix} m={m}")
    assert np.isfinite(y).all()
    del pw
    torch.cuda.empty_cache()
