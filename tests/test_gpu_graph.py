"""qpn_gemm captured in a HIP graph (torch.cuda.CUDAGraph): every replay,
with eager work and synchronizations in between, must reproduce the eager
result bit for bit, including the split-K path whose arrival counters each
call leaves at zero."""

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import gpu_quantize, say, to_dev, to_host
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,n,k,m", [("nvfp4", 5120, 4352, 8), ("fp8", 640, 5120, 4),
                                       ("nvfp4", 2048, 1024, 1)])
def test_graph_replay_matches_eager(fmt, n, k, m):
    say("graph replay", fmt, n, k, m)
    w = workloads.weights(n, k, 31)
    pw, _ = gpu_quantize(fmt, to_dev(w))
    x = to_dev(workloads.activations(m, k, 32))
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    ws = qt.new_workspace(pw, m)
    qt.gemm(x, pw, out=y, workspace=ws)
    eager = to_host(y).copy()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qt.gemm(x, pw, out=y, workspace=ws)
    for i in range(5):
        y.fill_(0)                              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y).view(np.uint16), eager.view(np.uint16)), i
    if ws is not None:
        assert not to_host(ws[:64]).any()


@pytest.mark.parametrize("stage", [1, 2])
def test_graph_replay_uneven_grid(stage):
    """The uneven-group grid (9 wavefronts, 5 workgroups sharing 45 n-tiles)
    captured in a graph: every replay gives the eager bits."""
    say("graph replay uneven", stage)
    n, k, m = 720, 1552, 12 if stage == 2 else 3
    w = workloads.weights(n, k, 51)
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    x = to_dev(workloads.activations(m, k, 52))
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    kw = dict(split_k=1, waves=9, k_slices=1, depth=2, x_stage=stage, whole_groups=5)
    assert qt.new_workspace(pw, m, **kw) is None
    qt.gemm(x, pw, out=y, **kw)
    eager = to_host(y).copy()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qt.gemm(x, pw, out=y, **kw)
    for i in range(5):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y).view(np.uint16), eager.view(np.uint16)), i


@pytest.mark.parametrize("split", [0, 3])
def test_graph_replay_fused_epilogues(split):
    """The SwiGLU and greedy-argmax epilogues captured together in one graph
    (the argmax's key slots and the split-K counters are left at zero by each
    call, so every replay reproduces the eager bits)."""
    say("graph replay epilogues", split)
    n, k, m = 2048, 2304, 5
    w = workloads.weights(n, k, 41)
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    x = to_dev(workloads.activations(m, k, 42))
    h = torch.empty((m, n // 2), dtype=torch.float16, device="cuda")
    idx = torch.empty(m, dtype=torch.int32, device="cuda")
    val = torch.empty(m, dtype=torch.float32, device="cuda")
    kw = dict(split_k=split) if split else {}
    ws_h = qt.new_workspace(pw, m, swiglu=True, **kw)
    ws_a = qt.argmax_workspace(pw, m, **kw)

    def run():
        qt.gemm_swiglu(x, pw, out=h, workspace=ws_h, **kw)
        qt.gemm_argmax(x, pw, idx=idx, val=val, workspace=ws_a, **kw)

    run()
    eager = (to_host(h).copy(), to_host(idx).copy(), to_host(val).copy())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(5):
        h.fill_(0)
        idx.fill_(-1)
        val.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(h).view(np.uint16), eager[0].view(np.uint16)), i
        assert np.array_equal(to_host(idx), eager[1]), i
        assert np.array_equal(to_host(val).view(np.uint32), eager[2].view(np.uint32)), i
    # 128 n-tile counters (512 B) and the control block are back at zero
    assert not to_host(ws_a[:512 + 64 * 16 * 8]).any()
