"""GPU parity of the offline kernels: absmax, the NVFP4/FP8 quantizers and
pack/unpack, all bit-exact against the oracle (integer and byte work)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from golden_io import load_case
from gpu_helpers import DEV, oracle_quantize, say, to_dev, to_host
import quantized_weight_skinny_amd as q
from quantized_weight_skinny_amd import QPN_ERR_BAD_CODE, QpnError
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu


def test_absmax_exact_and_nan():
    say("absmax")
    for n in (0, 1, 255, 4097, 1 << 20):
        v = workloads.weights(1, n, 5 + n)[0] if n else np.zeros(0, np.float32)
        got = to_host(qt.absmax(to_dev(v)))[0]
        assert got == (np.abs(v).max() if n else 0.0)
    v = np.ones(1000, np.float32)
    v[777] = np.nan
    assert np.isnan(to_host(qt.absmax(to_dev(v)))[0])


def test_quantize_nvfp4_hand_case():
    say("quantize nvfp4 hand case")
    case = load_case("nvfp4_hand_case.json")
    codes, scales, s_t = qt.quantize_nvfp4(to_dev(case["W"]))
    assert s_t == case["tensor_scale"]
    assert np.array_equal(to_host(codes), case["packed_codes"])
    assert np.array_equal(to_host(scales), case["block_scale_codes"])


def test_quantize_fp8_hand_case():
    say("quantize fp8 hand case")
    case = load_case("fp8_hand_case.json")
    codes, rs = qt.quantize_fp8(to_dev(case["W"]))
    assert np.array_equal(to_host(codes), case["codes"])
    assert np.array_equal(to_host(rs), case["row_scales"])


SHAPES = [(512, 1024), (37, 48), (16, 272), (100, 2320), (1, 16)]


def _edge_weights(n, k, seed):
    """Random weights with ties, zeros, signed zeros, subnormals and spikes."""
    rng = np.random.default_rng(seed)
    w = workloads.weights(n, k, seed)
    mask = rng.random((n, k))
    w[mask < 0.05] = 0.0
    w[(mask >= 0.05) & (mask < 0.08)] = -0.0
    w[(mask >= 0.08) & (mask < 0.10)] *= 1e-36          # fp32 subnormals
    w[(mask >= 0.10) & (mask < 0.12)] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], 1)[0]
    w[(mask >= 0.99)] *= 50.0
    w[0, :16] = 0.0                                        # an all-zero block
    return w.astype(np.float32)


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("edge", [False, True])
def test_quantize_nvfp4_matches_oracle(n, k, edge):
    say("quantize nvfp4", n, k, edge)
    w = _edge_weights(n, k, 31 + n) if edge else workloads.weights(n, k, 31 + n)
    codes, scales, s_t = qt.quantize_nvfp4(to_dev(w))
    rc, rsc, rst = oracle_quantize("nvfp4", w)
    assert np.float32(s_t) == rst
    assert np.array_equal(to_host(scales), rsc)
    assert np.array_equal(to_host(codes), oracle.pack_nibbles(rc))


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("edge", [False, True])
def test_quantize_fp8_matches_oracle(n, k, edge):
    say("quantize fp8", n, k, edge)
    w = _edge_weights(n, k, 41 + n) if edge else workloads.weights(n, k, 41 + n)
    codes, rs = qt.quantize_fp8(to_dev(w))
    rc, rrs = oracle_quantize("fp8", w)
    assert np.array_equal(to_host(rs), rrs)
    assert np.array_equal(to_host(codes), rc)


@pytest.mark.parametrize("matrix", ["gate_up", "down", "lm_head"])
def test_quantize_full_size_sampled_rows(matrix):
    """Whole 27B-shaped matrices quantized on the GPU; the oracle redoes a
    sample of rows (with its own tensor scale, which must agree)."""
    n, k = workloads.SHAPES[matrix]
    say("quantize full size", matrix, n, k)
    w = workloads.weights(n, k, workloads.seed_for("nvfp4_27b_m1", matrix, "W"))
    wd = to_dev(w)
    codes, scales, s_t = qt.quantize_nvfp4(wd)
    amax = np.abs(w).max()
    rows = np.unique(np.concatenate([[0, 1, n - 1], np.random.default_rng(1).integers(0, n, 40)]))
    rc, rsc, rst = oracle.quantize_nvfp4(w[rows], tensor_scale=oracle.nvfp4_tensor_scale(amax))
    assert np.float32(s_t) == rst
    sel = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(to_host(scales.index_select(0, sel)), rsc)
    assert np.array_equal(to_host(codes.index_select(0, sel)), oracle.pack_nibbles(rc))
    if matrix != "lm_head":
        c8, r8 = qt.quantize_fp8(wd)
        oc, ors = oracle.quantize_fp8(w[rows])
        assert np.array_equal(to_host(r8.index_select(0, sel)), ors)
        assert np.array_equal(to_host(c8.index_select(0, sel)), oc)
    del wd
    torch.cuda.empty_cache()


PACK_SHAPES = [(512, 1024), (17, 48), (33, 272), (16, 256), (1, 16), (130, 4112)]


@pytest.mark.parametrize("n,k", PACK_SHAPES)
def test_pack_unpack_nvfp4_round_trip(n, k):
    say("pack nvfp4", n, k)
    codes = workloads.random_nibble_bytes(n, k, n * 7 + k)
    # every byte value, valid or not, must survive the layout (check=False
    # skips the count of invalid scale codes, which has its own test)
    scales = workloads.random_block_scale_codes(n, k, n * 11 + k, lo=0, hi=0xFF)
    pw = qt.pack_nvfp4(to_dev(codes), to_dev(scales), 1.0, n, k, check=False)
    c2, s2 = qt.unpack(pw)
    assert np.array_equal(to_host(c2), codes)
    assert np.array_equal(to_host(s2), scales)
    # every padding byte (rows past n, columns past k) is zero
    raw = to_host(pw.packed)
    nt, ku = -(-n // 16), -(-k // 256)
    units = raw.reshape(ku, nt, 2304)  # K-unit-major: unit u of every n-tile, then u + 1
    lane = np.arange(64)
    r, g = lane % 16, lane // 16
    for t in range(nt):
        for u in range(ku):
            for h in range(2):
                vec = units[u, t, h * 1024:(h + 1) * 1024].reshape(64, 16)
                row = t * 16 + r
                k0 = u * 256 + g * 64 + h * 32
                dead = (row >= n) | (k0 >= k)
                assert not vec[dead].any()


@pytest.mark.parametrize("n,k", PACK_SHAPES)
def test_pack_unpack_fp8_round_trip(n, k):
    say("pack fp8", n, k)
    codes = workloads.random_fp8_codes(n, k, n * 13 + k)
    rs = np.ones(n, np.float32)
    pw = qt.pack_fp8(to_dev(codes), to_dev(rs), n, k)
    (c2,) = qt.unpack(pw)
    assert np.array_equal(to_host(c2), codes)


def _c_pack(fmt, codes, scales, n, k):
    """The C entry point itself (ctypes, no torch wrapper): (status, count)."""
    lib = q.lib()
    nbytes = q.qpn_packed_bytes(q.QPN_FMT_NVFP4 if fmt == "nvfp4" else q.QPN_FMT_FP8_E4M3, n, k)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    bad = torch.full((1,), 12345, dtype=torch.int32, device=DEV)   # the call clears it
    c = to_dev(codes)
    s = torch.cuda.current_stream().cuda_stream
    if fmt == "nvfp4":
        st = lib.qpn_pack_nvfp4(c.data_ptr(), to_dev(scales).data_ptr(), n, k, packed.data_ptr(), nbytes,
                                bad.data_ptr(), s)
    else:
        st = lib.qpn_pack_fp8(c.data_ptr(), n, k, packed.data_ptr(), nbytes, bad.data_ptr(), s)
    return st, int(to_host(bad)[0])


def test_c_pack_returns_bad_code():
    """qpn_pack_* report invalid E4M3 codes through their own status:
    QPN_ERR_BAD_CODE (-3) for NaN (0x7F, 0xFF) and sign-set block scales and
    for NaN FP8 weights, QPN_OK otherwise, with the count in the counter."""
    say("c pack bad code")
    n, k = 32, 512
    codes = workloads.random_nibble_bytes(n, k, 3)
    ok = workloads.random_block_scale_codes(n, k, 4)
    assert _c_pack("nvfp4", codes, ok, n, k) == (q.QPN_OK, 0)
    for bad_code in (0x7F, 0xFF, 0x80, 0xB8, 0xFE):
        sc = ok.copy()
        sc[5, 3] = bad_code
        assert _c_pack("nvfp4", codes, sc, n, k) == (q.QPN_ERR_BAD_CODE, 1), hex(bad_code)
    sc = ok.copy()
    sc[0, 0], sc[31, 31], sc[7, 2] = 0x7F, 0xFF, 0x80
    assert _c_pack("nvfp4", codes, sc, n, k) == (q.QPN_ERR_BAD_CODE, 3)
    f8 = workloads.random_fp8_codes(n, k, 5)
    f8 = np.where((f8 & 0x7F) == 0x7F, f8 ^ 1, f8).astype(np.uint8)
    assert _c_pack("fp8", f8, None, n, k) == (q.QPN_OK, 0)
    f8[1, 1], f8[2, 2] = 0x7F, 0xFF
    assert _c_pack("fp8", f8, None, n, k) == (q.QPN_ERR_BAD_CODE, 2)


def test_pack_counts_invalid_codes():
    say("pack invalid codes")
    n, k = 32, 512
    codes = workloads.random_nibble_bytes(n, k, 3)
    scales = workloads.random_block_scale_codes(n, k, 4)
    scales[3, 5] = 0x7F          # NaN
    scales[30, 31] = 0xFF        # NaN
    with pytest.raises(QpnError) as e:
        qt.pack_nvfp4(to_dev(codes), to_dev(scales), 1.0, n, k)
    assert e.value.status == QPN_ERR_BAD_CODE and ": 2 invalid" in str(e.value)
    # block scales are positive: sign-set codes (-0 included) are invalid too
    scales[0, 0] = 0x80
    scales[7, 2] = 0xB8
    scales[31, 0] = 0xFE
    with pytest.raises(QpnError) as e:
        qt.pack_nvfp4(to_dev(codes), to_dev(scales), 1.0, n, k)
    assert ": 5 invalid" in str(e.value)
    # the largest and smallest valid scales pass
    ok = workloads.random_block_scale_codes(n, k, 5)
    ok[0, 0], ok[1, 1], ok[2, 2] = 0x00, 0x7E, 0x01
    qt.pack_nvfp4(to_dev(codes), to_dev(ok), 1.0, n, k)
    f8 = workloads.random_fp8_codes(n, k, 5)
    f8[0, 0] = 0x7F
    with pytest.raises(QpnError):
        qt.pack_fp8(to_dev(f8), to_dev(np.ones(n, np.float32)), n, k)
