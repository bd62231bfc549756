"""Pins for oracle.mlp: torch's SiLU, closed-form identities of SiLU, and the
fused-epilogue bound checked against worst-case perturbations of g and u."""

import numpy as np
import torch

import oracle


def test_silu_matches_torch():
    g = np.concatenate([np.linspace(-40, 40, 4001), np.random.default_rng(0).standard_normal(1000) * 5,
                        [0.0, -0.0, 1e-30, -1e-30, 700.0, -700.0]])
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    assert np.allclose(oracle.silu(g), ref, rtol=1e-15, atol=1e-300)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    # sigma(ln 3) = 3/4
    assert abs(oracle.silu(np.log(3.0)) - 0.75 * np.log(3.0)) < 1e-15
    g = np.random.default_rng(1).standard_normal(1000) * 6
    # silu(g) - silu(-g) = g, since sigma(g) + sigma(-g) = 1
    assert np.allclose(oracle.silu(g) - oracle.silu(-g), g, rtol=0, atol=1e-13)
    # far tails: silu(g) -> g above, -> 0 below
    assert oracle.silu(50.0) == 50.0 and abs(oracle.silu(-50.0)) < 1e-19


def test_silu_slope_bound():
    g = np.linspace(-20, 20, 400001)
    s = 1 / (1 + np.exp(-g))
    d = s * (1 + g * (1 - s))
    assert np.abs(d).max() <= oracle.mlp.SILU_SLOPE_MAX
    assert np.abs(d).max() > oracle.mlp.SILU_SLOPE_MAX - 1e-3


def test_swiglu_halves_and_product():
    y = np.arange(12, dtype=np.float64).reshape(2, 6) - 5
    h = oracle.swiglu(y)
    assert h.shape == (2, 3)
    g, u = y[:, :3], y[:, 3:]
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.array_equal(h, ref)
    # a gate of zero silences the unit whatever the up value
    y2 = np.array([[0.0, 3.0]])
    assert oracle.swiglu(y2)[0, 0] == 0.0


def test_swiglu_tolerance_covers_worst_case_perturbations():
    rng = np.random.default_rng(2)
    m, n = 4, 4096
    y = rng.standard_normal((m, n)) * 3
    b = np.abs(y) + rng.random((m, n)) * 20
    tol = oracle.swiglu_tolerance(y, b)
    h = oracle.swiglu(y)
    t = oracle.tolerance(b)
    tg, tu = oracle.split_gate_up(t)
    g, u = oracle.split_gate_up(y)
    for sg in (-1, 1):
        for su in (-1, 1):
            hp = oracle.silu(g + sg * tg) * (u + su * tu)
            # the fp16 rounding of the perturbed result
            hp16 = hp.astype(np.float16).astype(np.float64)
            assert np.all(np.abs(hp16 - h) <= tol)
    # and the bound is not vacuous: within 10x of the largest such error
    assert np.median(tol / (np.abs(oracle.silu(g + tg) * (u + tu) - h) + 1e-12)) < 10


def test_down_tolerance_reduces_to_the_gemm_bound_for_an_exact_h():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((3, 64))
    w = rng.standard_normal((10, 64)) * 0.1
    b = np.abs(h) @ np.abs(w).T
    assert np.allclose(oracle.down_tolerance(h, np.zeros_like(h), w), oracle.tolerance(b), rtol=1e-15, atol=0)


def test_down_tolerance_covers_the_worst_perturbation_of_h():
    """For each output n the largest |sum_k w[n,k] e[k]| with |e| <= h_tol is
    reached at e = sign(w[n]) * h_tol; add the down GEMM's own bound on that
    perturbed input and the total must stay inside down_tolerance."""
    rng = np.random.default_rng(4)
    m, f, n = 2, 256, 12
    h = rng.standard_normal((m, f)) * 4
    h_tol = np.abs(rng.standard_normal((m, f))) * 0.05
    w = rng.standard_normal((n, f)) * 0.05
    y = h @ w.T
    bound = oracle.down_tolerance(h, h_tol, w)
    for j in range(n):
        for sgn in (-1, 1):
            e = sgn * np.sign(w[j]) * h_tol
            hp = h + e
            yp = hp @ w[j]
            gemm_bound = oracle.tolerance(np.abs(hp) @ np.abs(w[j]))
            assert np.all(np.abs(yp - y[:, j]) + gemm_bound <= bound[:, j] * (1 + 1e-12))
    # not vacuous: the perturbation term alone reaches most of the bound's first part
    assert np.all(h_tol @ np.abs(w).T <= bound)


def test_gated_mlp_matches_an_independent_torch_route():
    rng = np.random.default_rng(5)
    m, k, f, n = 3, 96, 40, 24
    x = rng.standard_normal((m, k)).astype(np.float16).astype(np.float64)
    wg = rng.standard_normal((2 * f, k)) * 0.1
    wd = rng.standard_normal((n, f)) * 0.1
    h, h_tol, y, y_tol = oracle.gated_mlp(x, wg, wd)
    tx, twg, twd = (torch.from_numpy(a) for a in (x, wg, wd))
    gu = tx @ twg.T
    th = torch.nn.functional.silu(gu[:, :f]) * gu[:, f:]
    ty = th @ twd.T
    assert np.allclose(h, th.numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(y, ty.numpy(), rtol=1e-12, atol=1e-14)
    assert h.shape == (m, f) and y.shape == (m, n) and h_tol.shape == h.shape and y_tol.shape == y.shape
    assert np.all(h_tol > 0) and np.all(y_tol > 1e-3)


def test_gated_mlp_one_hot_closed_form():
    """x = e_k picks column k of each weight: g, u are known numbers, so h is
    silu(g) * u exactly and y = W_down h."""
    k, f = 8, 4
    wg = np.zeros((2 * f, k))
    wg[:f, 2] = [1.0, -2.0, 0.0, 3.0]      # gate column 2
    wg[f:, 2] = [2.0, 1.0, 5.0, -1.0]      # up column 2
    wd = np.eye(f)[:3] * 2.0               # y = 2 h[:3]
    x = np.zeros((1, k))
    x[0, 2] = 1.0
    h, _, y, _ = oracle.gated_mlp(x, wg, wd)
    g = np.array([1.0, -2.0, 0.0, 3.0])
    u = np.array([2.0, 1.0, 5.0, -1.0])
    want = g / (1 + np.exp(-g)) * u
    assert np.allclose(h[0], want, rtol=1e-15, atol=0)
    assert h[0, 2] == 0.0
    assert np.allclose(y[0], 2.0 * want[:3], rtol=1e-15, atol=0)
