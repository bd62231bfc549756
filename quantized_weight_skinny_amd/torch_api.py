"""torch plumbing around the libqpn entry points.

torch supplies device memory and the current HIP stream; each helper passes
pointers to one C entry point of the library (see ``include/qpn.h``) and
returns the tensors it allocated. No arithmetic of the method happens here.
"""

import torch

from . import (
    QPN_EPILOGUE_ARGMAX,
    QPN_EPILOGUE_F32,
    QPN_EPILOGUE_NONE,
    QPN_EPILOGUE_SWIGLU,
    QPN_X_STAGE_AUTO,
    QPN_X_STAGE_FULL,
    QPN_X_STAGE_RING,
    QPN_ERR_BAD_CODE,
    QPN_FMT_FP8_E4M3,
    QPN_FMT_NVFP4,
    QpnError,
    make_weight,
    qpn_absmax_f32,
    qpn_fp8_absmax,
    qpn_requantize_fp8_nvfp4,
    qpn_gemm,
    qpn_gemm_argmax,
    qpn_gemm_f32,
    qpn_gemm_tuned,
    qpn_nvfp4_tensor_scale,
    qpn_pack_fp8,
    qpn_pack_nvfp4,
    qpn_packed_bytes,
    qpn_quantize_fp8,
    qpn_quantize_nvfp4,
    qpn_read_ceiling,
    qpn_read_ceiling_grid,
    qpn_unpack_fp8,
    qpn_unpack_nvfp4,
    qpn_workspace_bytes,
    qpn_workspace_bytes_tuned,
    make_launch,
    make_mlp_launch,
    qpn_mlp,
    qpn_mlp_workspace_bytes,
)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _cuda(t, dtype, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t


def _count(t, count, name):
    """The kernels read exactly `count` elements of t: refuse any other size."""
    if t.numel() != count:
        raise ValueError(f"{name} must hold {count} elements, not {t.numel()}")


def _activations(x, pw):
    """x fp16 [m, K] on the device, K the weight's (the kernels read m * K halves)."""
    _cuda(x, torch.float16, "x")
    if x.dim() != 2 or x.shape[1] != pw.k:
        raise ValueError(f"x must have shape (m, {pw.k}), not {tuple(x.shape)}")
    return x.shape[0]


def _output(out, shape, dtype, like, name="out"):
    """A new output tensor, or the caller's after checking that the kernel's
    writes fit it."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _cuda(out, dtype, name)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(out.shape)}")
    return out


class PackedWeight:
    """A packed [n, k] weight on the device plus its scales."""

    def __init__(self, fmt, n, k, packed, tensor_scale=1.0, row_scales=None):
        self.fmt, self.n, self.k = fmt, n, k
        self.packed = packed
        self.tensor_scale = float(tensor_scale)
        self.row_scales = row_scales

    def desc(self):
        rs = self.row_scales.data_ptr() if self.row_scales is not None else None
        return make_weight(self.fmt, self.n, self.k, self.packed.data_ptr(), self.tensor_scale, rs)

    @property
    def nbytes(self):
        """Bytes the GEMM streams for this weight (packed codes and scales,
        plus the fp32 row scales of FP8)."""
        extra = self.row_scales.numel() * 4 if self.row_scales is not None else 0
        return self.packed.numel() + extra


def _pack(call, bad, where, check):
    """Run a pack call; the C call itself returns QPN_ERR_BAD_CODE for invalid
    codes (after it has written every packed byte). check=False keeps the
    packed bytes anyway (layout round-trip tests of every byte value)."""
    try:
        call()
    except QpnError as e:
        if e.status != QPN_ERR_BAD_CODE:
            raise
        if check:
            count = int(bad.item())
            raise QpnError(QPN_ERR_BAD_CODE,
                           f"{where}: {count} invalid E4M3 code(s) (NaN, or a sign-set block scale)") from None


def pack_nvfp4(codes, block_scales, tensor_scale, n, k, check=True):
    """Canonical NVFP4 codes [n, k/2] + E4M3 block scales [n, k/16] -> PackedWeight."""
    _cuda(codes, torch.uint8, "codes")
    _cuda(block_scales, torch.uint8, "block_scales")
    _count(codes, n * (k // 2), "codes")
    _count(block_scales, n * (k // 16), "block_scales")
    nbytes = qpn_packed_bytes(QPN_FMT_NVFP4, n, k)
    packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=codes.device)
    bad = torch.zeros(1, dtype=torch.int32, device=codes.device)
    _pack(lambda: qpn_pack_nvfp4(codes.data_ptr(), block_scales.data_ptr(), n, k, packed.data_ptr(), nbytes,
                                 bad.data_ptr(), _stream()), bad, "qpn_pack_nvfp4", check)
    return PackedWeight(QPN_FMT_NVFP4, n, k, packed[:nbytes] if nbytes else packed, tensor_scale)


def pack_fp8(codes, row_scales, n, k, check=True):
    """Canonical E4M3 codes [n, k] + fp32 row scales [n] -> PackedWeight."""
    _cuda(codes, torch.uint8, "codes")
    _cuda(row_scales, torch.float32, "row_scales")
    _count(codes, n * k, "codes")
    _count(row_scales, n, "row_scales")
    nbytes = qpn_packed_bytes(QPN_FMT_FP8_E4M3, n, k)
    packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=codes.device)
    bad = torch.zeros(1, dtype=torch.int32, device=codes.device)
    _pack(lambda: qpn_pack_fp8(codes.data_ptr(), n, k, packed.data_ptr(), nbytes, bad.data_ptr(), _stream()), bad,
          "qpn_pack_fp8", check)
    return PackedWeight(QPN_FMT_FP8_E4M3, n, k, packed[:nbytes] if nbytes else packed, 1.0, row_scales)


def unpack(pw):
    """PackedWeight -> canonical tensors (codes, block scales) or (codes,)."""
    dev = pw.packed.device
    if pw.fmt == QPN_FMT_NVFP4:
        codes = torch.empty((pw.n, pw.k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((pw.n, pw.k // 16), dtype=torch.uint8, device=dev)
        qpn_unpack_nvfp4(pw.packed.data_ptr(), pw.packed.numel(), pw.n, pw.k, codes.data_ptr(),
                         scales.data_ptr(), _stream())
        return codes, scales
    codes = torch.empty((pw.n, pw.k), dtype=torch.uint8, device=dev)
    qpn_unpack_fp8(pw.packed.data_ptr(), pw.packed.numel(), pw.n, pw.k, codes.data_ptr(), _stream())
    return (codes,)


def absmax(w):
    """max |w| over a float32 CUDA tensor, computed by the library (returns a
    1-element device tensor)."""
    _cuda(w, torch.float32, "w")
    out = torch.empty(1, dtype=torch.float32, device=w.device)
    qpn_absmax_f32(w.data_ptr(), w.numel(), out.data_ptr(), _stream())
    return out


def nvfp4_tensor_scale(amax):
    return qpn_nvfp4_tensor_scale(float(amax))


def quantize_nvfp4(w, tensor_scale=None):
    """float32 W [n, k] on the device -> (codes [n, k/2], block scales [n, k/16], s_t)."""
    _cuda(w, torch.float32, "w")
    n, k = w.shape
    if tensor_scale is None:
        amax = absmax(w).item()
        if amax != amax or amax == float("inf"):
            raise ValueError("weights must be finite")
        tensor_scale = nvfp4_tensor_scale(amax)
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // 16), dtype=torch.uint8, device=w.device)
    qpn_quantize_nvfp4(w.data_ptr(), n, k, tensor_scale, codes.data_ptr(), scales.data_ptr(), _stream())
    return codes, scales, tensor_scale


def quantize_fp8(w):
    """float32 W [n, k] on the device -> (codes [n, k], row scales [n])."""
    _cuda(w, torch.float32, "w")
    n, k = w.shape
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    rs = torch.empty(n, dtype=torch.float32, device=w.device)
    qpn_quantize_fp8(w.data_ptr(), n, k, codes.data_ptr(), rs.data_ptr(), _stream())
    return codes, rs


def requantize_fp8_to_nvfp4(codes8, row_scales):
    """(codes [n, k/2], block scales [n, k/16], tensor scale) of an FP8 weight
    (uint8 codes [n, k], fp32 row scales [n]) converted to NVFP4 on the GPU;
    pack the result with pack_nvfp4."""
    _cuda(codes8, torch.uint8, "codes")
    _cuda(row_scales, torch.float32, "row_scales")
    n, k = codes8.shape
    _count(row_scales, n, "row_scales")
    amax = torch.empty(1, dtype=torch.float32, device=codes8.device)
    qpn_fp8_absmax(codes8.data_ptr(), row_scales.data_ptr(), n, k, amax.data_ptr(), _stream())
    s_t = qpn_nvfp4_tensor_scale(float(amax.item()))
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=codes8.device)
    scales = torch.empty((n, k // 16), dtype=torch.uint8, device=codes8.device)
    qpn_requantize_fp8_nvfp4(codes8.data_ptr(), row_scales.data_ptr(), n, k, s_t, codes.data_ptr(),
                             scales.data_ptr(), _stream())
    return codes, scales, s_t


def _launch(split_k=0, waves=0, depth=0, k_slices=0, epilogue=QPN_EPILOGUE_NONE, x_stage=0, whole_groups=0,
            valu_dot=0, block_columns=0):
    if split_k or waves or depth or k_slices or epilogue or x_stage or whole_groups or valu_dot or block_columns:
        return make_launch(split_k, waves, depth, k_slices, epilogue, x_stage, whole_groups, valu_dot, block_columns)
    return None


def workspace_bytes(pw, m, split_k=0, waves=0, depth=0, k_slices=0, swiglu=False, x_stage=0, whole_groups=0,
                    valu_dot=0, block_columns=0):
    launch = _launch(split_k, waves, depth, k_slices, QPN_EPILOGUE_SWIGLU if swiglu else QPN_EPILOGUE_NONE, x_stage,
                     whole_groups, valu_dot, block_columns)
    d = pw.desc()
    return qpn_workspace_bytes_tuned(d, m, launch) if launch is not None else qpn_workspace_bytes(d, m)


def new_workspace(pw, m, split_k=0, waves=0, depth=0, k_slices=0, swiglu=False, device="cuda", x_stage=0,
                  whole_groups=0, valu_dot=0, block_columns=0):
    """A zeroed workspace for gemm(pw) with m rows (None when none is needed)."""
    need = workspace_bytes(pw, m, split_k, waves, depth, k_slices, swiglu, x_stage, whole_groups, valu_dot,
                           block_columns)
    return torch.zeros(need, dtype=torch.uint8, device=device) if need else None


def _run(x, pw, out, workspace, launch, cols, dtype=torch.float16):
    m = _activations(x, pw)
    out = _output(out, (m, cols), dtype, x)
    d = pw.desc()
    need = qpn_workspace_bytes_tuned(d, m, launch) if launch is not None else qpn_workspace_bytes(d, m)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if need else 0
    if launch is not None:
        qpn_gemm_tuned(x.data_ptr(), d, out.data_ptr(), m, ws_ptr, ws_bytes, launch, _stream())
    else:
        qpn_gemm(x.data_ptr(), d, out.data_ptr(), m, ws_ptr, ws_bytes, _stream())
    return out


def gemm(x, pw, out=None, workspace=None, split_k=0, waves=0, depth=0, k_slices=0, x_stage=0, whole_groups=0,
         valu_dot=0, block_columns=0):
    """y[m, n] = x[m, k] @ dequant(W)^T in fp16 through qpn_gemm (any shape
    field set: qpn_gemm_tuned; valu_dot=1: the VALU packed-dot path;
    block_columns=1/2: the block-column MFMA path at m=1 on / off).

    A workspace, when one is needed and not given, is allocated zeroed per
    call; pass one from new_workspace() to reuse it across calls."""
    return _run(x, pw, out, workspace,
                _launch(split_k, waves, depth, k_slices, x_stage=x_stage, whole_groups=whole_groups,
                        valu_dot=valu_dot, block_columns=block_columns), pw.n)


def gemm_f32(x, pw, out=None, workspace=None, split_k=0, waves=0, depth=0, k_slices=0, x_stage=0, whole_groups=0):
    """y[m, n] = x[m, k] @ dequant(W)^T as fp32, not rounded (a row-parallel
    rank's partial sum): qpn_gemm_f32, or with any shape field set
    qpn_gemm_tuned with the F32 epilogue."""
    if not (split_k or waves or depth or k_slices or x_stage or whole_groups):
        m = _activations(x, pw)
        out = _output(out, (m, pw.n), torch.float32, x)
        d = pw.desc()
        need = qpn_workspace_bytes_tuned(d, m, make_launch(epilogue=QPN_EPILOGUE_F32))
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
        qpn_gemm_f32(x.data_ptr(), d, out.data_ptr(), m, workspace.data_ptr() if need else None,
                     workspace.numel() * workspace.element_size() if need else 0, _stream())
        return out
    launch = make_launch(split_k, waves, depth, k_slices, QPN_EPILOGUE_F32, x_stage, whole_groups)
    return _run(x, pw, out, workspace, launch, pw.n, torch.float32)


def gemm_swiglu(x, pw, out=None, workspace=None, split_k=0, waves=0, depth=0, k_slices=0, x_stage=0,
                whole_groups=0):
    """h[m, n/2] = silu(g) * u with [g | u] = x @ dequant(W)^T (W's first n/2
    rows are the gate projection): the SwiGLU epilogue of qpn_gemm_tuned
    (zero shape fields: the shape qpn_gemm_swiglu uses)."""
    launch = make_launch(split_k, waves, depth, k_slices, QPN_EPILOGUE_SWIGLU, x_stage, whole_groups)
    return _run(x, pw, out, workspace, launch, pw.n // 2)


def argmax_workspace(pw, m, split_k=0, waves=0, depth=0, k_slices=0, device="cuda", x_stage=0, whole_groups=0):
    """A zeroed workspace for gemm_argmax(pw) with up to m rows."""
    launch = make_launch(split_k, waves, depth, k_slices, QPN_EPILOGUE_ARGMAX, x_stage, whole_groups)
    return torch.zeros(qpn_workspace_bytes_tuned(pw.desc(), m, launch), dtype=torch.uint8, device=device)


def gemm_argmax(x, pw, idx=None, val=None, workspace=None, split_k=0, waves=0, depth=0, k_slices=0,
                x_stage=0, whole_groups=0):
    """(idx int32 [m], val fp32 [m]): each row's largest logit of
    x @ dequant(W)^T and its index, through qpn_gemm_argmax."""
    m = _activations(x, pw)
    launch = make_launch(split_k, waves, depth, k_slices, QPN_EPILOGUE_ARGMAX, x_stage, whole_groups)
    d = pw.desc()
    need = qpn_workspace_bytes_tuned(d, m, launch)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    idx = _output(idx, (m,), torch.int32, x, "idx")
    val = _output(val, (m,), torch.float32, x, "val")
    qpn_gemm_argmax(x.data_ptr(), d, idx.data_ptr(), val.data_ptr(), m, workspace.data_ptr(),
                    workspace.numel() * workspace.element_size(), launch, _stream())
    return idx, val


def mlp_workspace(gate_up, down, m, fused=0, down_depth=0, stream_after=0, device="cuda"):
    """A zeroed workspace for mlp(gate_up, down) with up to m rows."""
    launch = make_mlp_launch(fused, down_depth, stream_after)
    return torch.zeros(qpn_mlp_workspace_bytes(gate_up.desc(), down.desc(), m, launch), dtype=torch.uint8,
                       device=device)


def mlp(x, gate_up, down, h=None, y=None, workspace=None, fused=0, down_depth=0, stream_after=0):
    """(h, y, launches): h = SwiGLU of x @ dequant(W_gu)^T (fp16 [m, n_gu/2])
    and y = h @ dequant(W_dn)^T (fp16 [m, n_dn]) through qpn_mlp, in one
    launch where possible (fused=1: only that, fused=2: two launches);
    launches is the number of kernels the call enqueued."""
    m = _activations(x, gate_up)
    if down.k != gate_up.n // 2:
        raise ValueError(f"down must have k = {gate_up.n // 2}, not {down.k}")
    launch = make_mlp_launch(fused, down_depth, stream_after)
    need = qpn_mlp_workspace_bytes(gate_up.desc(), down.desc(), m, launch)
    if need == 0:
        raise QpnError(-2, "qpn_mlp_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    h = _output(h, (m, down.k), torch.float16, x, "h")
    y = _output(y, (m, down.n), torch.float16, x, "y")
    n = qpn_mlp(x.data_ptr(), gate_up.desc(), down.desc(), h.data_ptr(), y.data_ptr(), m, workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), launch, _stream())
    return h, y, n


def mlp_status(workspace, gate_up, down, m, fused=0, down_depth=0, stream_after=0):
    """The status word of the control block of a workspace that mlp() used
    with these arguments (1: a wait of the one-launch form ran past its
    bound; that call's results are undefined). Reads device memory, so it
    synchronizes."""
    need = qpn_mlp_workspace_bytes(gate_up.desc(), down.desc(), m, make_mlp_launch(fused, down_depth, stream_after))
    word = workspace.view(torch.uint8)[need - 256 + 8: need - 256 + 12]
    return int(word.cpu().view(torch.int32)[0])


def read_ceiling(buf, grid=0, sink=None, loads=0):
    """One pass of the read-only streaming kernel over a uint8 CUDA tensor
    (``loads`` 16-byte loads in flight per thread: 2, 4 or 8; 0 = 4)."""
    g = grid or qpn_read_ceiling_grid()
    if sink is None:
        sink = torch.empty(g * 4, dtype=torch.int32, device=buf.device)
    _count(sink, sink.numel(), "sink")
    if sink.numel() < g * 4:
        raise ValueError(f"sink must hold {g * 4} words")
    qpn_read_ceiling(buf.data_ptr(), buf.numel() - buf.numel() % 16, sink.data_ptr(), g, loads, _stream())
    return sink
