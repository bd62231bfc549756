"""GPU parity of the fused MLP (qpn_mlp: gate_up with SwiGLU, then down, in one
launch where possible) against the oracle's gated MLP: h within the SwiGLU
bound and y within the bound that the two GEMM bounds imply
(oracle.gated_mlp). Also: the one-launch and two-launch forms agree bit for
bit where their launch shapes agree, the control counters return to zero, and
a captured graph replays it correctly."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, gpu_quantize, oracle_quantize, say, to_dev, to_host
import quantized_weight_skinny_amd as q
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu


def _dequant(fmt, parts):
    if fmt == "nvfp4":
        codes, sc, s_t = parts
        return oracle.dequantize_nvfp4(codes, sc, s_t)
    codes, rs = parts
    return oracle.dequantize_fp8(codes, rs)


def _check(h, y, ref, what):
    h_ref, h_tol, y_ref, y_tol = ref
    assert np.isfinite(h).all() and np.isfinite(y).all(), what
    eh = np.abs(h.astype(np.float64) - h_ref)
    assert np.all(eh <= h_tol), f"{what}: h {int((eh > h_tol).sum())} outside, worst {(eh - h_tol).max():.3g}"
    ey = np.abs(y.astype(np.float64) - y_ref)
    assert np.all(ey <= y_tol), f"{what}: y {int((ey > y_tol).sum())} outside, worst {(ey - y_tol).max():.3g}"


def _weights(fmt_up, fmt_dn, f, k, n, seed):
    """Quantized gate_up [2f, k] and down [n, f]: packed on the device and
    dequantized by the oracle (each side quantizes the same seeded fp32)."""
    wg = workloads.weights(2 * f, k, seed)
    wd = workloads.weights(n, f, seed + 1)
    pg, _ = gpu_quantize(fmt_up, to_dev(wg))
    pd, _ = gpu_quantize(fmt_dn, to_dev(wd))
    return pg, pd, _dequant(fmt_up, oracle_quantize(fmt_up, wg)), _dequant(fmt_dn, oracle_quantize(fmt_dn, wd))


def _seeded_nvfp4(n, k, seed):
    """Seeded canonical NVFP4 codes with moderate block scales (the oracle
    only dequantizes them), packed on the device."""
    codes = workloads.random_nibble_bytes(n, k, seed)
    scales = workloads.random_block_scale_codes(n, k, seed + 1, lo=0x20, hi=0x40)
    s_t = np.float32(2.0 ** -6)
    pw = qt.pack_nvfp4(to_dev(codes), to_dev(scales), float(s_t), n, k)
    return pw, oracle.dequantize_nvfp4(oracle.unpack_nibbles(codes), scales, s_t)


def _ordered(a):
    """fp16 values as integers in value order (fp16 ulps apart = integers
    apart; -0 and +0 are both 0)."""
    b = a.view(np.uint16).astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - b, b)


# (F, K, N): F the hidden width of the MLP (h columns), K the model width, N
# down's output rows; ragged tiles and K tails included.
SHAPES = [(64, 256, 64), (528, 1024, 100), (1024, 272, 512), (2048, 1024, 320)]


@pytest.mark.parametrize("f,k,n", SHAPES)
@pytest.mark.parametrize("m", [1, 2])
@pytest.mark.parametrize("fused", [1, 2])
def test_mlp_parity(fused, m, f, k, n):
    say("mlp", fused, m, f, k, n)
    pg, pd, wg, wd = _weights("nvfp4", "nvfp4", f, k, n, seed=4000 + f + k + n)
    x = workloads.activations(m, k, 4100 + m)
    h, y, launches = qt.mlp(to_dev(x), pg, pd, fused=fused)
    assert launches == fused
    _check(to_host(h), to_host(y), oracle.gated_mlp(x, wg, wd), f"fused={fused} m={m} f={f} k={k} n={n}")


@pytest.mark.parametrize("m", [3, 8, 16])
def test_mlp_more_rows(m):
    """More rows: automatic takes two launches; one launch (down's K range
    cut to fit its stage) where the grid still fits the device, else
    refused; either way within the bounds."""
    say("mlp rows", m)
    f, k, n = 2048, 512, 256
    pg, pd, wg, wd = _weights("nvfp4", "nvfp4", f, k, n, seed=4200 + m)
    x = workloads.activations(m, k, 4300 + m)
    for fused in (0, 1):
        try:
            h, y, launches = qt.mlp(to_dev(x), pg, pd, fused=fused)
        except q.QpnError as e:  # one launch may not fit the device at these rows
            assert fused == 1 and e.status == q.QPN_ERR_UNSUPPORTED
            continue
        assert launches == (2 if fused == 0 else 1)
        _check(to_host(h), to_host(y), oracle.gated_mlp(x, wg, wd), f"fused={fused} m={m}")


def test_mlp_grid_too_large_for_one_launch():
    """A gate_up of 8192 n-tiles needs more workgroups than the device holds
    at once: the automatic call takes two launches and a call that asks for
    one is refused (QPN_ERR_UNSUPPORTED, nothing enqueued)."""
    say("mlp grid too large")
    f, k, n = 65536, 256, 64
    pg, wg = _seeded_nvfp4(2 * f, k, 4900)
    pd, wd = _seeded_nvfp4(n, f, 4910)
    x = workloads.activations(1, k, 4920)
    with pytest.raises(q.QpnError) as e:
        qt.mlp(to_dev(x), pg, pd, fused=1)
    assert e.value.status == q.QPN_ERR_UNSUPPORTED
    h, y, launches = qt.mlp(to_dev(x), pg, pd)
    assert launches == 2
    _check(to_host(h), to_host(y), oracle.gated_mlp(x, wg, wd), "grid too large")


@pytest.mark.parametrize("fmts", [("fp8", "nvfp4"), ("nvfp4", "fp8"), ("fp8", "fp8")])
def test_mlp_other_formats_take_two_launches(fmts):
    say("mlp formats", fmts)
    f, k, n = 528, 512, 96
    pg, pd, wg, wd = _weights(*fmts, f, k, n, seed=4400)
    x = workloads.activations(2, k, 4401)
    h, y, launches = qt.mlp(to_dev(x), pg, pd)
    assert launches == 2
    _check(to_host(h), to_host(y), oracle.gated_mlp(x, wg, wd), f"formats {fmts}")


@pytest.mark.parametrize("down_depth", [3, 4, 6, 8])
@pytest.mark.parametrize("stream_after", [-1, 0, 1, 1000000])
def test_mlp_launch_options(down_depth, stream_after):
    """Every consumer depth, and consumers that stream at once, after half
    the producers (automatic), after the first, and only after all of them
    (a count past the producers is clamped)."""
    say("mlp options", down_depth, stream_after)
    f, k, n = 1024, 512, 256
    pg, pd, wg, wd = _weights("nvfp4", "nvfp4", f, k, n, seed=4500)
    x = workloads.activations(1, k, 4501)
    h, y, launches = qt.mlp(to_dev(x), pg, pd, fused=1, down_depth=down_depth, stream_after=stream_after)
    assert launches == 1
    _check(to_host(h), to_host(y), oracle.gated_mlp(x, wg, wd), f"depth {down_depth} after {stream_after}")


def test_mlp_counters_return_to_zero_and_calls_repeat():
    """Three calls on one workspace (rows 1, 2, 1): each is right, the status
    word stays 0 and the control block's counters are zero again after each
    call (so is the rest: these shapes split no K range)."""
    say("mlp repeat")
    f, k, n = 1024, 1024, 512
    pg, pd, wg, wd = _weights("nvfp4", "nvfp4", f, k, n, seed=4600)
    ws = qt.mlp_workspace(pg, pd, 2, fused=1)
    for i, m in enumerate([1, 2, 1]):
        x = workloads.activations(m, k, 4601 + i)
        h, y, launches = qt.mlp(to_dev(x), pg, pd, workspace=ws, fused=1)
        assert launches == 1
        _check(to_host(h), to_host(y), oracle.gated_mlp(x, wg, wd), f"call {i} m={m}")
        assert qt.mlp_status(ws, pg, pd, 2, fused=1) == 0
        assert int(torch.count_nonzero(ws)) == 0, f"call {i}: workspace not left zero"


def test_mlp_graph_replays():
    """The one-launch form captured in a graph (no memset inside): replays
    with eager work between them match the eager call bit for bit."""
    say("mlp graph")
    f, k, n = 2048, 1024, 320
    pg, pd, _, _ = _weights("nvfp4", "nvfp4", f, k, n, seed=4700)
    x = to_dev(workloads.activations(1, k, 4701))
    ws = qt.mlp_workspace(pg, pd, 1, fused=1)
    h0, y0, _ = qt.mlp(x, pg, pd, workspace=ws, fused=1)
    h0, y0 = to_host(h0), to_host(y0)
    h = torch.empty((1, f), dtype=torch.float16, device=DEV)
    y = torch.empty((1, n), dtype=torch.float16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qt.mlp(x, pg, pd, h=h, y=y, workspace=ws, fused=1)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qt.mlp(x, pg, pd, h=h, y=y, workspace=ws, fused=1)
    for r in range(4):
        h.zero_()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(h).view(np.uint16), h0.view(np.uint16)), f"replay {r}: h"
        assert np.array_equal(to_host(y).view(np.uint16), y0.view(np.uint16)), f"replay {r}: y"
        qt.gemm(x, pg)  # eager work between replays
        torch.cuda.synchronize()
    assert qt.mlp_status(ws, pg, pd, 1, fused=1) == 0


@pytest.mark.parametrize("m", [1, 2])
def test_mlp_full_size_all_outputs(m):
    """The 27B MLP (gate_up 34816 x 5120, down 5120 x 17408, NVFP4) at the
    bench's rows, in one launch: every h and y element against the oracle;
    y equal bit for bit to the down GEMM run alone on that h; and (M = 1,
    where gate_up takes the same launch shape in both forms) h equal to the
    gate_up GEMM's SwiGLU epilogue run alone but for rare elements one fp16
    ulp apart. At M = 2 the forms cut gate_up differently, so their fp32 sums
    differ in order and only the oracle bound applies."""
    n_gu, k = workloads.SHAPES["gate_up"]
    n_dn, f = workloads.SHAPES["down"]
    assert f == n_gu // 2
    say("mlp full size", m)
    pg, wg = _seeded_nvfp4(n_gu, k, 4800)
    pd, wd = _seeded_nvfp4(n_dn, f, 4810)
    x = workloads.activations(m, k, workloads.seed_for("nvfp4_27b_mlp", "gate_up", "x") + m)
    xd = to_dev(x)
    h1, y1, launches = qt.mlp(xd, pg, pd, fused=1)
    assert launches == 1
    y_alone = to_host(qt.gemm(h1, pd))
    h_alone = to_host(qt.gemm_swiglu(xd, pg))
    h1, y1 = to_host(h1), to_host(y1)
    del pg, pd
    torch.cuda.empty_cache()
    _check(h1, y1, oracle.gated_mlp(x, wg, wd), f"full size m={m} one launch")
    assert np.array_equal(y1.view(np.uint16), y_alone.view(np.uint16))
    if m == 1:  # the same launch shape for gate_up in both forms
        diff = _ordered(h1) - _ordered(h_alone)
        assert np.abs(diff).max() <= 1 and np.count_nonzero(diff) <= h1.size // 1000, np.count_nonzero(diff)
