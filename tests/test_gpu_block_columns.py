"""GPU parity of the block-column path (one activation row of NVFP4 weights):
the matrix cores' 16 output columns carry the 16 K-blocks of a 256-element
unit, and each E4M3 block scale multiplies an fp32 block sum. The result is
the same dot product summed in another order, so it is held to the oracle's
bound, and to exact results where the arithmetic is exact (one-hot
activations, negation, scale doubling, row permutation, repeat calls)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, assert_within_tolerance, gpu_quantize, oracle_quantize, oracle_y, say, to_dev, to_host
import quantized_weight_skinny_amd as q
from quantized_weight_skinny_amd import torch_api as qt

pytestmark = pytest.mark.gpu

ON, OFF = 1, 2
SHAPES = [(512, 1024), (37, 48), (100, 272), (16, 4096), (33, 2304), (300, 5120), (64, 17408), (1, 16)]


def _case(n, k, seed):
    w = workloads.weights(n, k, seed)
    x = workloads.activations(1, k, seed + 1)
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    y_ref, b = oracle_y("nvfp4", x, oracle_quantize("nvfp4", w))
    return pw, to_dev(x), y_ref, b


@pytest.mark.parametrize("n,k", SHAPES)
def test_block_columns_parity(n, k):
    say("block columns", n, k)
    pw, x, y_ref, b = _case(n, k, 3000 + n + k)
    plan = q.qpn_gemm_plan(pw.desc(), 1, q.make_launch(block_columns=ON))
    assert plan.block_columns == ON
    y_on = to_host(qt.gemm(x, pw, block_columns=ON))
    y_off = to_host(qt.gemm(x, pw, block_columns=OFF))
    assert_within_tolerance(y_on, y_ref, b, f"block columns on {n}x{k}")
    assert_within_tolerance(y_off, y_ref, b, f"block columns off {n}x{k}")


LAUNCHES = [dict(split_k=1, waves=4, depth=2, k_slices=1), dict(split_k=3, waves=8, depth=3, k_slices=2),
            dict(split_k=2, waves=8, depth=4, k_slices=4), dict(split_k=7, waves=4, depth=6, k_slices=1),
            dict(split_k=1, waves=8, depth=8, k_slices=8), dict(split_k=4, whole_groups=5, waves=4, depth=3,
                                                                k_slices=2),
            dict(split_k=1, waves=8, depth=3, k_slices=4)]


@pytest.mark.parametrize("kw", LAUNCHES)
def test_block_columns_launch_shapes(kw):
    """Split-K, whole groups, K slices and every stream depth (the zero region
    the B operand reads scales with the depth)."""
    say("block columns launch", kw)
    pw, x, y_ref, b = _case(300, 3328, 55)
    y = to_host(qt.gemm(x, pw, block_columns=ON, x_stage=qt.QPN_X_STAGE_FULL, **kw))
    assert_within_tolerance(y, y_ref, b, f"block columns {kw}")
    ws = qt.new_workspace(pw, 1, x_stage=qt.QPN_X_STAGE_FULL, block_columns=ON, **kw)
    again = to_host(qt.gemm(x, pw, workspace=ws, block_columns=ON, x_stage=qt.QPN_X_STAGE_FULL, **kw))
    assert np.array_equal(again.view(np.uint16), y.view(np.uint16))


def test_block_columns_one_hot_is_exact():
    """x = e_k: one block sum is one weight's E2M1 value, times its block
    scale, times a power-of-two tensor scale: every weight reads back exactly,
    including every block of a unit and the last element of a ragged K."""
    say("block columns one hot")
    for n, k, s_t in ((64, 512, 1.0), (20, 272, 0.25), (33, 1040, 2.0)):
        codes = workloads.random_nibble_bytes(n, k, 5)
        scales = workloads.random_block_scale_codes(n, k, 6)
        pw = qt.pack_nvfp4(to_dev(codes), to_dev(scales), s_t, n, k)
        wdq = oracle.dequantize_nvfp4(oracle.unpack_nibbles(codes), scales, s_t)
        for kk in sorted({0, 1, 7, 8, 15, 16, 31, 63, 64, 100, 127, 128, 200, 255, k - 1}):
            if kk >= k:
                continue
            x = np.zeros((1, k), np.float16)
            x[0, kk] = 1.0
            y = to_host(qt.gemm(to_dev(x), pw, block_columns=ON))
            assert np.array_equal(y[0].astype(np.float64), wdq[:, kk]), (n, k, kk)


def _f32_block_columns(x, pw, split_k=0, k_slices=0, waves=0):
    """The fp32-output GEMM at one row with block columns (qpn_gemm_tuned)."""
    launch = q.make_launch(split_k, waves, 0, k_slices, epilogue=q.QPN_EPILOGUE_F32, x_stage=q.QPN_X_STAGE_FULL,
                           block_columns=ON)
    need = q.qpn_workspace_bytes_tuned(pw.desc(), 1, launch)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    y = torch.empty((1, pw.n), dtype=torch.float32, device=DEV)
    q.qpn_gemm_tuned(x.data_ptr(), pw.desc(), y.data_ptr(), 1, ws.data_ptr() if need else None, need, launch,
                     torch.cuda.current_stream().cuda_stream)
    return to_host(y)


def test_block_columns_closed_forms():
    """Negation and repeat calls give the same bits; doubling the tensor scale
    doubles the fp32 output; permuting W's rows permutes y's columns."""
    say("block columns closed forms")
    n, k = 304, 2304
    w = to_dev(workloads.weights(n, k, 61))
    x = to_dev(workloads.activations(1, k, 62))
    codes, scales, s_t = qt.quantize_nvfp4(w)
    perm = np.random.default_rng(63).permutation(n)
    pt = torch.from_numpy(perm).to(DEV)
    pw = qt.pack_nvfp4(codes, scales, s_t, n, k)
    pw2 = qt.pack_nvfp4(codes, scales, 2 * s_t, n, k)
    pwp = qt.pack_nvfp4(codes[pt].contiguous(), scales[pt].contiguous(), s_t, n, k)
    for kw in ({}, dict(split_k=3), dict(k_slices=4, waves=8)):
        y = to_host(qt.gemm(x, pw, block_columns=ON, **kw))
        assert np.array_equal(to_host(qt.gemm(x, pw, block_columns=ON, **kw)).view(np.uint16), y.view(np.uint16))
        assert np.array_equal(to_host(qt.gemm(-x, pw, block_columns=ON, **kw)), -y)
        yp = to_host(qt.gemm(x, pwp, block_columns=ON, **kw))
        assert np.array_equal(yp.view(np.uint16), y[:, perm].view(np.uint16)), kw
        f1 = _f32_block_columns(x, pw, **kw)
        assert np.array_equal(_f32_block_columns(x, pw2, **kw), 2 * f1), kw


def test_block_columns_epilogues():
    """The fp32, SwiGLU and greedy-argmax epilogues at one row with block
    columns."""
    say("block columns epilogues")
    n, k = 512, 2048
    w = workloads.weights(n, k, 71)
    x = workloads.activations(1, k, 72)
    pw, _ = gpu_quantize("nvfp4", to_dev(w))
    parts = oracle_quantize("nvfp4", w)
    y_ref, b = oracle_y("nvfp4", x, parts)
    xd = to_dev(x)
    full = q.QPN_X_STAGE_FULL
    for epi, out, dtype in ((q.QPN_EPILOGUE_F32, (1, n), torch.float32), (q.QPN_EPILOGUE_SWIGLU, (1, n // 2),
                                                                           torch.float16)):
        launch = q.make_launch(epilogue=epi, x_stage=full, block_columns=ON)
        assert q.qpn_gemm_plan(pw.desc(), 1, launch).block_columns == ON
        y = torch.empty(out, dtype=dtype, device=DEV)
        q.qpn_gemm_tuned(xd.data_ptr(), pw.desc(), y.data_ptr(), 1, None, 0, launch,
                         torch.cuda.current_stream().cuda_stream)
        got = to_host(y).astype(np.float64)
        if epi == q.QPN_EPILOGUE_F32:
            assert_within_tolerance(got, y_ref, b, "f32")
        else:
            assert np.all(np.abs(got - oracle.swiglu(y_ref)) <= oracle.swiglu_tolerance(y_ref, b))
    launch = q.make_launch(epilogue=q.QPN_EPILOGUE_ARGMAX, x_stage=full, block_columns=ON)
    ws = torch.zeros(q.qpn_workspace_bytes_tuned(pw.desc(), 1, launch), dtype=torch.uint8, device=DEV)
    idx = torch.empty(1, dtype=torch.int32, device=DEV)
    q.qpn_gemm_argmax(xd.data_ptr(), pw.desc(), idx.data_ptr(), None, 1, ws.data_ptr(), ws.numel(), launch,
                      torch.cuda.current_stream().cuda_stream)
    assert oracle.argmax_candidates(y_ref, b)[0, int(to_host(idx)[0])]


@pytest.mark.parametrize("name", ["gate_up", "down", "qkv", "o_proj", "lm_head"])
def test_block_columns_full_size(name):
    """The 27B shapes at one row with block columns, every output column
    against the oracle (computed in row chunks)."""
    n, k = workloads.SHAPES[name]
    say("block columns full size", name, n, k)
    w = workloads.weights(n, k, workloads.seed_for("block_columns", name, "W"))
    x = workloads.activations(1, k, workloads.seed_for("block_columns", name, "x"))
    wd = to_dev(w)
    codes, scales, s_t = qt.quantize_nvfp4(wd)
    pw = qt.pack_nvfp4(codes, scales, s_t, n, k)
    del wd
    y = to_host(qt.gemm(to_dev(x), pw, block_columns=ON, x_stage=qt.QPN_X_STAGE_FULL))
    c = oracle.unpack_nibbles(to_host(codes))
    sc = to_host(scales)
    step = 8192
    for r0 in range(0, n, step):
        y_ref, b = oracle.gemm_nvfp4(x, c[r0:r0 + step], sc[r0:r0 + step], s_t)
        assert_within_tolerance(y[:, r0:r0 + step], y_ref, b, f"{name} rows {r0}..")
