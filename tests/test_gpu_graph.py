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
