"""GPU parity of the gate_up GEMM with the SwiGLU epilogue (through the C ABI)
against the oracle: h = silu(g) * u on the float64 GEMM result, within the
bound that the GEMM's own bound on g and u implies (oracle.swiglu_tolerance)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, gpu_quantize, oracle_quantize, oracle_y, say, to_dev, to_host
import quantized_weight_skinny_amd as q
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu


def _check(h, y_ref, b, what):
    h_ref = oracle.swiglu(y_ref)
    tol = oracle.swiglu_tolerance(y_ref, b)
    err = np.abs(h.astype(np.float64) - h_ref)
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} outside the bound, worst {(err - tol).max():.3g}"
    assert np.isfinite(h).all()


def _parity(fmt, m, n, k, seed, **kw):
    w = workloads.weights(n, k, seed)
    x = workloads.activations(m, k, seed + 1)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    h = to_host(qt.gemm_swiglu(to_dev(x), pw, **kw))
    assert h.shape == (m, n // 2)
    y_ref, b = oracle_y(fmt, x, oracle_quantize(fmt, w))
    _check(h, y_ref, b, f"{fmt} m={m} n={n} k={k} {kw}")
    return h


SHAPES = [(64, 1024), (96, 272), (1056, 2304), (512, 5120)]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 3, 8, 16])
def test_swiglu_parity(fmt, m, n, k):
    say("swiglu", fmt, m, n, k)
    _parity(fmt, m, n, k, seed=3000 + n + k + m)


LAUNCHES = [dict(split_k=2, waves=8, depth=2, k_slices=2), dict(split_k=3, waves=4, depth=3, k_slices=1),
            dict(split_k=1, waves=8, depth=3, k_slices=4), dict(split_k=5, waves=8, depth=4, k_slices=1),
            dict(split_k=1, waves=4, depth=2, k_slices=2),
            # the ring activation stage (x_stage 2)
            dict(split_k=1, waves=8, depth=3, k_slices=2, x_stage=2), dict(split_k=3, waves=4, depth=2, k_slices=1, x_stage=2),
            dict(split_k=1, waves=8, depth=4, k_slices=4, x_stage=2),
            # leading groups whole, the others split
            dict(split_k=3, waves=4, depth=2, k_slices=1, x_stage=2, whole_groups=5),
            dict(split_k=2, waves=8, depth=3, k_slices=2, x_stage=1, whole_groups=3)]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("kw", LAUNCHES, ids=lambda d: "-".join(str(v) for v in d.values()))
def test_swiglu_launch_shapes(fmt, kw):
    """Both epilogue paths: in-workgroup (one K range) and the split-K
    reduction of the last workgroup, with ragged groups (33 gate tiles)."""
    say("swiglu launch", fmt, kw)
    _parity(fmt, 5, 1056, 2304, seed=77, **kw)


def test_swiglu_entry_point_matches_tuned_auto_and_is_deterministic():
    say("swiglu abi")
    n, k, m = 512, 1024, 4
    w = workloads.weights(n, k, 5)
    x = to_dev(workloads.activations(m, k, 6))
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    h1 = qt.gemm_swiglu(x, pw)
    ws_bytes = q.qpn_workspace_bytes_tuned(pw.desc(), m, q.make_launch(epilogue=q.QPN_EPILOGUE_SWIGLU))
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    h2 = torch.empty((m, n // 2), dtype=torch.float16, device=DEV)
    q.qpn_gemm_swiglu(x.data_ptr(), pw.desc(), h2.data_ptr(), m, ws.data_ptr(), ws.numel(),
                      torch.cuda.current_stream().cuda_stream)
    a, b = to_host(h1), to_host(h2)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(to_host(qt.gemm_swiglu(x, pw)).view(np.uint16), a.view(np.uint16))


def test_swiglu_of_zero_gate_and_one_hot_rows():
    """x = e_k: g and u are single decoded weights (exact), so h is
    silu(g) * u of exactly known values, up to fp32 silu and fp16 rounding."""
    say("swiglu one hot")
    n, k = 64, 256
    codes = workloads.random_fp8_codes(n, k, 7)
    rs = np.full(n, 0.5, np.float32)
    pw = qt.pack_fp8(to_dev(codes), to_dev(rs), n, k)
    wdq = oracle.dequantize_fp8(codes, rs)
    ks = [0, 5, 100, 255]
    x = np.zeros((len(ks), k), np.float16)
    for i, kk in enumerate(ks):
        x[i, kk] = 1.0
    h = to_host(qt.gemm_swiglu(to_dev(x), pw)).astype(np.float64)
    for i, kk in enumerate(ks):
        g, u = wdq[: n // 2, kk], wdq[n // 2:, kk]
        want = oracle.silu(g) * u
        assert np.all(np.abs(h[i] - want) <= 2.0 ** -10 * np.abs(want) + 2.0 ** -24)
        assert np.all(h[i][g == 0] == 0)


@pytest.mark.parametrize("m", [1, 8])
def test_swiglu_full_size_gate_up(m):
    """The 27B gate_up (34816 x 5120 NVFP4) with the fused epilogue: on
    quantized weights the oracle recomputes sampled h columns from their gate
    and up rows; on seeded canonical codes it recomputes every h column."""
    n, k = workloads.SHAPES["gate_up"]
    say("swiglu full size", m)
    wl = "nvfp4_27b_mlp"
    w = workloads.weights(n, k, workloads.seed_for(wl, "gate_up", "W"))
    x = workloads.activations(m, k, workloads.seed_for(wl, "gate_up", "x"))
    wd = to_dev(w)
    pw, _ = gpu_quantize("nvfp4", wd)
    del wd
    h = to_host(qt.gemm_swiglu(to_dev(x), pw))
    half = n // 2
    cols = np.unique(np.concatenate([np.arange(16), np.arange(half - 16, half),
                                     np.random.default_rng(m).integers(0, half, 64)]))
    rows = np.concatenate([cols, cols + half])
    s_t = oracle.nvfp4_tensor_scale(np.abs(w).max())
    parts = oracle.quantize_nvfp4(w[rows], tensor_scale=s_t)
    y_ref, b = oracle.gemm_nvfp4(x, *parts)
    _check(h[:, cols], y_ref, b, f"gate_up swiglu m={m}")
    del pw
    # every h column, on seeded canonical codes (the oracle only dequantizes)
    codes = workloads.random_nibble_bytes(n, k, 17 + m)
    scales = workloads.random_block_scale_codes(n, k, 18 + m, lo=0x20, hi=0x40)
    pw = qt.pack_nvfp4(to_dev(codes), to_dev(scales), 2.0 ** -6, n, k)
    h = to_host(qt.gemm_swiglu(to_dev(x), pw))
    for c0 in range(0, half, 8192):
        cols = np.arange(c0, min(half, c0 + 8192))
        rows = np.concatenate([cols, cols + half])
        y_ref, b = oracle.gemm_nvfp4(x, oracle.unpack_nibbles(codes[rows]), scales[rows], np.float32(2.0 ** -6))
        _check(h[:, cols], y_ref, b, f"gate_up swiglu m={m} columns {c0}..")
    del pw
    torch.cuda.empty_cache()
