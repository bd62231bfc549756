"""GPU parity of qpn_gemm_f32, the fp32 output (through the C ABI), against the
float64 oracle, and its relation to qpn_gemm's fp16 output.

It is the same accumulator as qpn_gemm without the final rounding, so the bar
is:
- rounding y32 to fp16 gives qpn_gemm's bits (same launch shape), except where
  y32 lies exactly halfway between two fp16 values: qpn_gemm rounds the scaled
  accumulator to fp16 in one step, y32 is that product rounded to fp32 first,
  and there qpn_gemm's value is either neighbour;
- |y32 - y_ref| <= gamma(K + 64) * sum_k |x * w|, gamma(n) = n u / (1 - n u),
  u = 2^-24: the decoded weights and their products with fp16 activations are
  exact in fp32, so the error is that of fp32 sums along chains of at most K
  additions plus the K-slice and split-range adds and the scale;
- most outputs are not fp16 values (nothing rounded them to fp16)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, gpu_quantize, oracle_quantize, oracle_y, say, to_dev, to_host
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _fp32_bound(b, k):
    n = k + 64
    return n * U32 / (1 - n * U32) * b


def _same_as_fp16(y32, y16, what):
    """qpn_gemm's output is y32 rounded to fp16, up to double rounding at ties."""
    h = y32.astype(np.float16)
    diff = h.view(np.uint16) != y16.view(np.uint16)
    if diff.any():
        a, c, v = h[diff], y16[diff], y32[diff].astype(np.float64)
        adjacent = np.nextafter(a, c) == c
        halfway = (a.astype(np.float64) + c.astype(np.float64)) / 2 == v
        assert np.all(adjacent & halfway), (what, int(diff.sum()), v[~(adjacent & halfway)][:4])


def _check(y32, y16, y_ref, b, k, what):
    assert y32.dtype == np.float32 and y16.dtype == np.float16
    _same_as_fp16(y32, y16, what)
    err = np.abs(y32.astype(np.float64) - y_ref)
    tol = _fp32_bound(b, k)
    bad = ~(err <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the fp32 bound; first at {i}: "
                             f"gpu={y32[i]!r} ref={y_ref[i]!r} tol={tol[i]!r}")
    if k >= 48 and y32.size >= 64:
        not_half = np.mean(y32.astype(np.float16).astype(np.float32) != y32)
        assert not_half > 0.5, (what, not_half)


def _case(fmt, m, n, k, seed, **kw):
    w = workloads.weights(n, k, seed)
    x = workloads.activations(m, k, seed + 1)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    xd = to_dev(x)
    y32 = to_host(qt.gemm_f32(xd, pw, **kw))
    y16 = to_host(qt.gemm(xd, pw, **kw))
    y_ref, b = oracle_y(fmt, x, oracle_quantize(fmt, w))
    _check(y32, y16, y_ref, b, k, f"{fmt} m={m} n={n} k={k} {kw}")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k", [(512, 1024), (37, 48), (100, 272), (33, 2304), (300, 5120)])
@pytest.mark.parametrize("m", [1, 3, 8, 16])
def test_f32_output_small(fmt, m, n, k):
    say("gemm f32", fmt, m, n, k)
    _case(fmt, m, n, k, seed=3000 + n + k + m)


RING = qt.QPN_X_STAGE_RING
F32_LAUNCHES = [
    dict(split_k=3, waves=8, depth=4, k_slices=1),
    dict(split_k=2, waves=4, depth=3, k_slices=2),
    dict(split_k=4, waves=4, depth=2, k_slices=1, whole_groups=1),
    dict(split_k=1, waves=8, depth=3, k_slices=4),
    dict(split_k=2, waves=8, depth=3, k_slices=2, x_stage=RING),
    dict(split_k=1, waves=4, depth=2, k_slices=1, x_stage=RING),
]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("kw", F32_LAUNCHES, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_f32_output_launch_shapes(fmt, kw):
    n, k, m = 160, 1792, 5
    say("gemm f32 tuned", fmt, kw)
    _case(fmt, m, n, k, seed=91, **kw)


# Row-parallel shapes (K is what tensor parallelism splits): the per-GPU
# o_proj and down of 4-way TP, and the whole down matrix.
ROW_PARALLEL = [("nvfp4", "o_proj_tp4", 1), ("nvfp4", "o_proj_tp4", 8), ("nvfp4", "down_tp4", 1),
                ("nvfp4", "down_tp4", 8), ("nvfp4", "down", 1), ("nvfp4", "down", 8), ("fp8", "down", 4)]


@pytest.mark.parametrize("fmt,matrix,m", ROW_PARALLEL)
def test_f32_output_full_size_sampled(fmt, matrix, m):
    """Full-size matrices in the automatic launch shape; the oracle recomputes
    a sample of output columns, the fp16 identity covers every output."""
    n, k = workloads.SHAPES[matrix]
    say("gemm f32 full size", fmt, matrix, m, n, k)
    wl = "decode_step_27b"
    w = workloads.weights(n, k, workloads.seed_for(wl, matrix, "W"))
    x = workloads.activations(m, k, workloads.seed_for(wl, matrix, "x"))
    wd = to_dev(w)
    pw, _ = gpu_quantize(fmt, wd)
    del wd
    xd = to_dev(x)
    y32 = to_host(qt.gemm_f32(xd, pw))
    y16 = to_host(qt.gemm(xd, pw))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                     np.random.default_rng(n + m + 1).integers(0, n, 96)]))
    if fmt == "nvfp4":
        parts = oracle.quantize_nvfp4(w[cols], tensor_scale=oracle.nvfp4_tensor_scale(np.abs(w).max()))
    else:
        parts = oracle.quantize_fp8(w[cols])
    y_ref, b = oracle_y(fmt, x, parts)
    _same_as_fp16(y32, y16, f"{fmt} {matrix} m={m} all outputs")
    _check(y32[:, cols], y16[:, cols], y_ref, b, k, f"{fmt} {matrix} m={m}")
    del pw
    torch.cuda.empty_cache()


def test_f32_output_edge_cases():
    say("gemm f32 edge cases")
    # K = 0: the empty sum is +0 in every output
    pw = qt.pack_nvfp4(torch.zeros((4, 0), dtype=torch.uint8, device=DEV),
                       torch.zeros((4, 0), dtype=torch.uint8, device=DEV), 1.0, 4, 0)
    y = torch.full((2, 4), 7.0, dtype=torch.float32, device=DEV)
    qt.gemm_f32(torch.zeros((2, 0), dtype=torch.float16, device=DEV), pw, out=y)
    assert not to_host(y).any()
    # a caller's output buffer: written exactly in place, guard words untouched
    n, k, m = 50, 512, 3
    w = workloads.weights(n, k, 14)
    pw, _ = gpu_quantize("fp8", to_dev(w))
    buf = torch.full((m * n + 64,), 12345.0, dtype=torch.float32, device=DEV)
    x = to_dev(workloads.activations(m, k, 15))
    qt.gemm_f32(x, pw, out=buf[:m * n].view(m, n))
    assert np.all(to_host(buf[m * n:]) == np.float32(12345.0))
    y16 = to_host(qt.gemm(x, pw))
    _same_as_fp16(to_host(buf[:m * n]).reshape(m, n), y16, "in place")
    # outputs of the wrong type or shape are refused before any launch
    with pytest.raises(ValueError):
        qt.gemm_f32(x, pw, out=torch.empty((m, n), dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        qt.gemm_f32(x, pw, out=torch.empty((m, n - 1), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        qt.gemm(x, pw, out=torch.empty((m + 1, n), dtype=torch.float16, device=DEV))
