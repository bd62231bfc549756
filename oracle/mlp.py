"""SwiGLU between the two MLP GEMMs, in float64 (test infrastructure only).

The pages run the GEMM inside a dense decoder's MLP ([P3] "What I actually
built": the kernels are measured at the decoder's own shapes), but they do
not describe the MLP itself. The plainest reading of a gated MLP with a fused
gate_up projection is taken here: the gate_up weight is the row concatenation
[W_gate; W_up], so the first N/2 outputs of y = x @ W_gate_up^T are the gate
g and the last N/2 the up projection u, and the down projection's input is

    h[m, j] = silu(g[m, j]) * u[m, j],    silu(g) = g / (1 + exp(-g)).

``swiglu`` writes that out on the oracle's exact float64 y. A kernel that
fuses it into the GEMM's epilogue computes it from its fp32 accumulators and
rounds h once to fp16; ``swiglu_tolerance`` is the acceptance bound that
follows from the GEMM's own bound on g and u (derived at the function).
"""

import numpy as np

SILU_SLOPE_MAX = 1.0999  # max |d silu / dg| over the reals (about 1.0998 at g = 2.40)


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def split_gate_up(y):
    """(gate, up) halves of a gate_up GEMM output y[M, N], N even."""
    y = np.asarray(y, dtype=np.float64)
    if y.shape[-1] % 2:
        raise ValueError("gate_up output needs an even number of columns")
    half = y.shape[-1] // 2
    return y[..., :half], y[..., half:]


def swiglu(y):
    """h[M, N/2] = silu(gate) * up from a gate_up GEMM output y[M, N]."""
    g, u = split_gate_up(y)
    return silu(g) * u


def swiglu_tolerance(y, b):
    """Per-element bound on |h_gpu - h| when g and u each come within the
    GEMM bound t = 2e-3 * b + 1e-3 of their exact values.

    With |dg| <= t_g and |du| <= t_u:
      |silu(g + dg) (u + du) - silu(g) u|
        <= |silu(g)| t_u + |u| L t_g + L t_g t_u        (L = max |silu'|)
    plus the single rounding of h to fp16 (2^-11 |h|, with |h| bounded by
    the perturbed value) and the fp32 evaluation of silu and the product
    (a few fp32 ulps, covered by 1e-6 relative), plus the fp16 subnormal
    spacing for results near zero.
    """
    g, u = split_gate_up(y)
    bg, bu = split_gate_up(b)
    tg = 2e-3 * bg + 1e-3
    tu = 2e-3 * bu + 1e-3
    sg = np.abs(silu(g))
    lin = sg * tu + np.abs(u) * SILU_SLOPE_MAX * tg + SILU_SLOPE_MAX * tg * tu
    hmax = sg * np.abs(u) + lin
    return lin + (2.0 ** -11 + 1e-6) * hmax + 2.0 ** -24


def down_tolerance(h, h_tol, w_down):
    """Per-element bound on |y_gpu - y| for the down GEMM y = h W_down^T
    (y[M, N], h[M, F], w_down the dequantized float64 W_down[N, F]) when the
    GPU's h differs from the exact h by at most h_tol elementwise.

    The down GEMM runs on the GPU's own h, h' = h + e with |e| <= h_tol, and
    comes within the GEMM bound of its exact result on that input:
        |y_gpu - h' W^T| <= 2e-3 * sum_k |w[n,k] h'[k]| + 1e-3,
    while |h' W^T - h W^T| = |sum_k w[n,k] e[k]| <= sum_k |w[n,k]| h_tol[k].
    With |h'| <= |h| + h_tol:
        |y_gpu - y| <= |W| h_tol + 2e-3 * |W| (|h| + h_tol) + 1e-3
    (matrix products over k, written on the transposed layout).
    """
    h = np.asarray(h, dtype=np.float64)
    h_tol = np.asarray(h_tol, dtype=np.float64)
    aw = np.abs(np.asarray(w_down, dtype=np.float64))
    return h_tol @ aw.T + 2e-3 * ((np.abs(h) + h_tol) @ aw.T) + 1e-3


def gated_mlp(x, w_gate_up, w_down):
    """(h, h_tol, y, y_tol) of the gated MLP on activations x[M, K]:
    g | u = x W_gate_up^T exactly (float64), h = silu(g) * u, y = h W_down^T,
    with the acceptance bounds of a GPU that computes the two GEMMs within
    2e-3 * sum|w x| + 1e-3 and rounds h once to fp16 (swiglu_tolerance and
    down_tolerance). w_gate_up [2F, K] and w_down [N, F] are the dequantized
    float64 weights."""
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_gate_up, dtype=np.float64)
    y_gu = x @ wg.T
    b_gu = np.abs(x) @ np.abs(wg).T
    h = swiglu(y_gu)
    h_tol = swiglu_tolerance(y_gu, b_gu)
    wd = np.asarray(w_down, dtype=np.float64)
    return h, h_tol, h @ wd.T, down_tolerance(h, h_tol, wd)

