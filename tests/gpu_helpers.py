"""Shared setup for the GPU parity tests: seeded inputs from workloads.py go to
both the HIP path (through the C ABI) and the oracle; nothing flows from the
HIP path into an expected value."""

import sys

import numpy as np
import torch

import oracle
import workloads
from quantized_weight_skinny_amd import QPN_FMT_FP8_E4M3, QPN_FMT_NVFP4
from quantized_weight_skinny_amd import torch_api as qt

DEV = "cuda:0"


def say(*args):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print("[gpu case]", *args, file=sys.stderr, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_quantize(fmt, w_dev):
    """Quantize + pack on the device; returns (PackedWeight, canonical parts)."""
    n, k = w_dev.shape
    if fmt == "nvfp4":
        codes, scales, s_t = qt.quantize_nvfp4(w_dev)
        pw = qt.pack_nvfp4(codes, scales, s_t, n, k)
        return pw, (codes, scales, s_t)
    codes, rs = qt.quantize_fp8(w_dev)
    pw = qt.pack_fp8(codes, rs, n, k)
    return pw, (codes, rs)


def oracle_quantize(fmt, w, tensor_scale=None):
    if fmt == "nvfp4":
        codes, sc, s_t = oracle.quantize_nvfp4(w, tensor_scale)
        return codes, sc, s_t
    return oracle.quantize_fp8(w)


def oracle_y(fmt, x, parts):
    if fmt == "nvfp4":
        codes, sc, s_t = parts
        return oracle.gemm_nvfp4(x, codes, sc, s_t)
    codes, rs = parts
    return oracle.gemm_fp8(x, codes, rs)


def assert_within_tolerance(y_gpu, y_ref, b, what=""):
    """|y_gpu - y_ref| <= 2e-3 * sum|w*x| + 1e-3, element by element."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    tol = oracle.tolerance(b)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs out of tolerance; first at {tuple(i)}: "
            f"gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r} tol={tol[tuple(i)]!r}")


FMT_CODE = {"nvfp4": QPN_FMT_NVFP4, "fp8": QPN_FMT_FP8_E4M3}
