"""qpn_gemm_noalloc, the entry point for callers that cannot allocate: through
the C ABI, against qpn_gemm with a caller workspace (same launch, same
kernels: the same bits), on calls in a row on one stream, each later one
smaller, so the shared scratch carries counters and partials from the call
before; one case also against the oracle."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, assert_within_tolerance, gpu_quantize, oracle_quantize, oracle_y, say, to_dev, to_host
import quantized_weight_skinny_amd as q
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu


def _noalloc(x, pw, m):
    y = torch.empty((m, pw.n), dtype=torch.float16, device=DEV)
    st = q.lib().qpn_gemm_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.byref(pw.desc()),
                                  ctypes.c_void_p(y.data_ptr()), m,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == q.QPN_OK, q.qpn_status_string(st)
    return y


def _with_workspace(x, pw, m):
    y = torch.empty((m, pw.n), dtype=torch.float16, device=DEV)
    need = q.qpn_workspace_bytes(pw.desc(), m)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    st = q.lib().qpn_gemm(ctypes.c_void_p(x.data_ptr()), ctypes.byref(pw.desc()), ctypes.c_void_p(y.data_ptr()), m,
                          ctypes.c_void_p(ws.data_ptr() if need else None), ctypes.c_size_t(need),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == q.QPN_OK, q.qpn_status_string(st)
    return y


def _weight(fmt, name, wl="no_alloc"):
    n, k = workloads.SHAPES[name]
    w = workloads.weights(n, k, workloads.seed_for(wl, name, "W"))
    wd = to_dev(w)
    pw, _ = gpu_quantize(fmt, wd)
    del wd
    return pw, w


def test_noalloc_matches_the_workspace_entry_point_on_calls_in_a_row():
    # largest first: gate_up at 4 rows (split tail partials, 2.2 MB of
    # scratch), then down at 8 rows (split 3), then FP8 down at 2 rows, then
    # launches with no split at all (gate_up at 16 rows on the uneven grid,
    # the output head at one row)
    cases = [("nvfp4", "gate_up", 4), ("nvfp4", "down", 8), ("fp8", "down", 2), ("nvfp4", "gate_up", 16),
             ("nvfp4", "lm_head", 1)]
    needs = []
    for fmt, name, m in cases:
        say("no alloc", fmt, name, m)
        pw, _ = _weight(fmt, name)
        need = q.qpn_workspace_bytes(pw.desc(), m)
        assert need <= q.QPN_NOALLOC_SCRATCH_BYTES
        needs.append(need)
        x = to_dev(workloads.activations(m, pw.k, workloads.seed_for("no_alloc", name, f"x{m}")))
        y_ref = to_host(_with_workspace(x, pw, m))
        for _ in range(2):   # the second call finds the scratch as the first left it
            y = to_host(_noalloc(x, pw, m))
            assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16)), (fmt, name, m)
        del pw
        torch.cuda.empty_cache()
    assert needs[0] > needs[1] > needs[2] > 0 and needs[3] == needs[4] == 0


def test_noalloc_against_the_oracle_and_a_smaller_second_call():
    for fmt, (n, k), m in (("nvfp4", (1000, 17408), 8), ("fp8", (300, 17408), 3)):
        say("no alloc oracle", fmt, n, k, m)
        w = workloads.weights(n, k, 7 + m)
        x = workloads.activations(m, k, 8 + m)
        pw, _ = gpu_quantize(fmt, to_dev(w))
        assert q.qpn_workspace_bytes(pw.desc(), m) > 0
        y = to_host(_noalloc(to_dev(x), pw, m))
        y_ref, b = oracle_y(fmt, x, oracle_quantize(fmt, w))
        assert_within_tolerance(y, y_ref, b, f"no alloc {fmt} {n}x{k} m={m}")


def test_noalloc_refuses_what_does_not_fit():
    say("no alloc limits")
    # 1024 x 2^20 at 16 rows splits K into hundreds of ranges: more
    # partials than the scratch holds; refused before any launch
    w = q.make_weight(q.QPN_FMT_NVFP4, 1024, 1 << 20, 16)
    assert q.qpn_workspace_bytes(w, 16) > q.QPN_NOALLOC_SCRATCH_BYTES
    y = torch.empty(16, dtype=torch.uint8, device=DEV)
    st = q.lib().qpn_gemm_noalloc(ctypes.c_void_p(16), ctypes.byref(w), ctypes.c_void_p(y.data_ptr()), 16, None)
    assert st == q.QPN_ERR_BUFFER_TOO_SMALL
