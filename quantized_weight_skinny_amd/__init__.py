"""Python binding of libqpn.so, the weight-streaming skinny GEMM for MI355X.

``quantized_weight_skinny_amd.qpn_*`` mirror the C entry points of
``include/qpn.h`` one for one: integer device pointers and sizes in, the
qpn_status code checked (a negative status raises ``QpnError``). Nothing here
computes: every step runs in the HIP kernels of the library. The torch-facing
helpers in ``quantized_weight_skinny_amd.torch_api`` only allocate device
memory and pass pointers and the current stream.

The library is loaded on first use; if it has not been built the call fails
loudly (there is no fallback path).
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqpn.so")

QPN_OK = 0
QPN_ERR_INVALID_ARG = -1
QPN_ERR_UNSUPPORTED = -2
QPN_ERR_BAD_CODE = -3
QPN_ERR_BUFFER_TOO_SMALL = -4
QPN_ERR_HIP = -5

QPN_FMT_NVFP4 = 1
QPN_FMT_FP8_E4M3 = 2
QPN_MAX_M = 16

QPN_EPILOGUE_NONE = 0
QPN_EPILOGUE_SWIGLU = 1
QPN_EPILOGUE_ARGMAX = 2
QPN_EPILOGUE_F32 = 3
QPN_X_STAGE_AUTO = 0
QPN_X_STAGE_FULL = 1
QPN_X_STAGE_RING = 2


class QpnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {qpn_status_string(status)} ({status})")


class qpn_launch(ctypes.Structure):
    _fields_ = [
        ("split_k", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32),
        ("depth", ctypes.c_int32),
        ("k_slices", ctypes.c_int32),
        ("epilogue", ctypes.c_int32),
        ("x_stage", ctypes.c_int32),
        ("whole_groups", ctypes.c_int32),
        ("valu_dot", ctypes.c_int32),
        ("block_columns", ctypes.c_int32),
    ]


class qpn_mlp_launch(ctypes.Structure):
    _fields_ = [
        ("fused", ctypes.c_int32),
        ("down_depth", ctypes.c_int32),
        ("stream_after", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class qpn_weight(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("packed", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_float),
        ("row_scales", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_W = ctypes.POINTER(qpn_weight)
_L = ctypes.POINTER(qpn_launch)
_ML = ctypes.POINTER(qpn_mlp_launch)

# name -> (restype, argtypes); the declarations of include/qpn.h
SIGNATURES = {
    "qpn_status_string": (ctypes.c_char_p, [_I32]),
    "qpn_packed_bytes": (_SZ, [_I32, _I64, _I64]),
    "qpn_pack_nvfp4": (_I32, [_P, _P, _I64, _I64, _P, _SZ, _P, _P]),
    "qpn_pack_fp8": (_I32, [_P, _I64, _I64, _P, _SZ, _P, _P]),
    "qpn_unpack_nvfp4": (_I32, [_P, _SZ, _I64, _I64, _P, _P, _P]),
    "qpn_unpack_fp8": (_I32, [_P, _SZ, _I64, _I64, _P, _P]),
    "qpn_absmax_f32": (_I32, [_P, _I64, _P, _P]),
    "qpn_nvfp4_tensor_scale": (_F, [_F]),
    "qpn_quantize_nvfp4": (_I32, [_P, _I64, _I64, _F, _P, _P, _P]),
    "qpn_quantize_fp8": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "qpn_fp8_absmax": (_I32, [_P, _P, _I64, _I64, _P, _P]),
    "qpn_requantize_fp8_nvfp4": (_I32, [_P, _P, _I64, _I64, _F, _P, _P, _P]),
    "qpn_workspace_bytes": (_SZ, [_W, _I32]),
    "qpn_workspace_bytes_tuned": (_SZ, [_W, _I32, _L]),
    "qpn_gemm_plan": (_I32, [_W, _I32, _L, _L]),
    "qpn_gemm": (_I32, [_P, _W, _P, _I32, _P, _SZ, _P]),
    "qpn_gemm_noalloc": (_I32, [_P, _W, _P, _I32, _P]),
    "qpn_gemm_tuned": (_I32, [_P, _W, _P, _I32, _P, _SZ, _L, _P]),
    "qpn_gemm_swiglu": (_I32, [_P, _W, _P, _I32, _P, _SZ, _P]),
    "qpn_gemm_f32": (_I32, [_P, _W, _P, _I32, _P, _SZ, _P]),
    "qpn_gemm_argmax": (_I32, [_P, _W, _P, _P, _I32, _P, _SZ, _L, _P]),
    "qpn_mlp_workspace_bytes": (_SZ, [_W, _W, _I32, _ML]),
    "qpn_mlp": (_I32, [_P, _W, _W, _P, _P, _I32, _P, _SZ, _ML, ctypes.POINTER(_I32), _P]),
    "qpn_read_ceiling": (_I32, [_P, _SZ, _P, _I32, _I32, _P]),
    "qpn_read_ceiling_grid": (_I32, []),
}

_lib = None


def lib():
    """The loaded libqpn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m quantized_weight_skinny_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status, where):
    if status != QPN_OK:
        raise QpnError(status, where)
    return status


def qpn_status_string(status):
    return lib().qpn_status_string(status).decode()


def qpn_packed_bytes(fmt, n, k):
    return lib().qpn_packed_bytes(fmt, n, k)


def qpn_pack_nvfp4(codes, block_scales, n, k, packed, packed_bytes, bad_codes, stream):
    return _check(lib().qpn_pack_nvfp4(codes, block_scales, n, k, packed, packed_bytes, bad_codes, stream),
                  "qpn_pack_nvfp4")


def qpn_pack_fp8(codes, n, k, packed, packed_bytes, bad_codes, stream):
    return _check(lib().qpn_pack_fp8(codes, n, k, packed, packed_bytes, bad_codes, stream), "qpn_pack_fp8")


def qpn_unpack_nvfp4(packed, packed_bytes, n, k, codes, block_scales, stream):
    return _check(lib().qpn_unpack_nvfp4(packed, packed_bytes, n, k, codes, block_scales, stream),
                  "qpn_unpack_nvfp4")


def qpn_unpack_fp8(packed, packed_bytes, n, k, codes, stream):
    return _check(lib().qpn_unpack_fp8(packed, packed_bytes, n, k, codes, stream), "qpn_unpack_fp8")


def qpn_absmax_f32(x, count, out, stream):
    return _check(lib().qpn_absmax_f32(x, count, out, stream), "qpn_absmax_f32")


def qpn_nvfp4_tensor_scale(amax):
    return lib().qpn_nvfp4_tensor_scale(amax)


def qpn_quantize_nvfp4(w, n, k, tensor_scale, codes, block_scales, stream):
    return _check(lib().qpn_quantize_nvfp4(w, n, k, tensor_scale, codes, block_scales, stream),
                  "qpn_quantize_nvfp4")


def qpn_quantize_fp8(w, n, k, codes, row_scales, stream):
    return _check(lib().qpn_quantize_fp8(w, n, k, codes, row_scales, stream), "qpn_quantize_fp8")


def qpn_fp8_absmax(codes, row_scales, n, k, out, stream):
    return _check(lib().qpn_fp8_absmax(codes, row_scales, n, k, out, stream), "qpn_fp8_absmax")


def qpn_requantize_fp8_nvfp4(fp8_codes, row_scales, n, k, tensor_scale, codes, block_scales, stream):
    return _check(lib().qpn_requantize_fp8_nvfp4(fp8_codes, row_scales, n, k, tensor_scale, codes, block_scales,
                                                 stream), "qpn_requantize_fp8_nvfp4")


def make_weight(fmt, n, k, packed, tensor_scale=1.0, row_scales=None):
    return qpn_weight(fmt, 0, n, k, packed, tensor_scale, row_scales)


def qpn_workspace_bytes(weight, m):
    return lib().qpn_workspace_bytes(ctypes.byref(weight), m)


def make_launch(split_k=0, waves_per_group=0, depth=0, k_slices=0, epilogue=QPN_EPILOGUE_NONE,
                x_stage=QPN_X_STAGE_AUTO, whole_groups=0, valu_dot=0, block_columns=0):
    return qpn_launch(split_k, waves_per_group, depth, k_slices, epilogue, x_stage, whole_groups, valu_dot,
                      block_columns)


def qpn_workspace_bytes_tuned(weight, m, launch):
    return lib().qpn_workspace_bytes_tuned(ctypes.byref(weight), m,
                                           ctypes.byref(launch) if launch is not None else None)


def qpn_gemm_plan(weight, m, launch=None):
    """The resolved launch shape (a qpn_launch) qpn_gemm_tuned would use."""
    out = qpn_launch()
    _check(lib().qpn_gemm_plan(ctypes.byref(weight), m, ctypes.byref(launch) if launch is not None else None,
                               ctypes.byref(out)), "qpn_gemm_plan")
    return out


def qpn_gemm(x, weight, y, m, workspace, workspace_bytes, stream):
    return _check(lib().qpn_gemm(x, ctypes.byref(weight), y, m, workspace, workspace_bytes, stream), "qpn_gemm")


def qpn_gemm_tuned(x, weight, y, m, workspace, workspace_bytes, launch, stream):
    return _check(lib().qpn_gemm_tuned(x, ctypes.byref(weight), y, m, workspace, workspace_bytes,
                                       ctypes.byref(launch) if launch is not None else None, stream),
                  "qpn_gemm_tuned")


def qpn_gemm_swiglu(x, weight, h, m, workspace, workspace_bytes, stream):
    return _check(lib().qpn_gemm_swiglu(x, ctypes.byref(weight), h, m, workspace, workspace_bytes, stream),
                  "qpn_gemm_swiglu")


QPN_NOALLOC_SCRATCH_BYTES = 16 << 20


def qpn_gemm_noalloc(x, weight, y, m, stream):
    return _check(lib().qpn_gemm_noalloc(x, ctypes.byref(weight), y, m, stream), "qpn_gemm_noalloc")


def qpn_gemm_f32(x, weight, y, m, workspace, workspace_bytes, stream):
    return _check(lib().qpn_gemm_f32(x, ctypes.byref(weight), y, m, workspace, workspace_bytes, stream),
                  "qpn_gemm_f32")


def qpn_gemm_argmax(x, weight, idx, val, m, workspace, workspace_bytes, launch, stream):
    return _check(lib().qpn_gemm_argmax(x, ctypes.byref(weight), idx, val, m, workspace, workspace_bytes,
                                        ctypes.byref(launch) if launch is not None else None, stream),
                  "qpn_gemm_argmax")


def make_mlp_launch(fused=0, down_depth=0, stream_after=0):
    return qpn_mlp_launch(fused, down_depth, stream_after, 0)


def qpn_mlp_workspace_bytes(gate_up, down, m, launch=None):
    return lib().qpn_mlp_workspace_bytes(ctypes.byref(gate_up), ctypes.byref(down), m,
                                         ctypes.byref(launch) if launch is not None else None)


def qpn_mlp(x, gate_up, down, h, y, m, workspace, workspace_bytes, launch, stream):
    """Returns the number of kernels the call enqueued (1 or 2)."""
    n = ctypes.c_int32(0)
    _check(lib().qpn_mlp(x, ctypes.byref(gate_up), ctypes.byref(down), h, y, m, workspace, workspace_bytes,
                         ctypes.byref(launch) if launch is not None else None, ctypes.byref(n), stream), "qpn_mlp")
    return n.value


def qpn_read_ceiling(buf, nbytes, sink, grid, loads, stream):
    return _check(lib().qpn_read_ceiling(buf, nbytes, sink, grid, loads, stream), "qpn_read_ceiling")


def qpn_read_ceiling_grid():
    return lib().qpn_read_ceiling_grid()
