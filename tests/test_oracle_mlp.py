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
