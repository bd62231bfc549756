"""Benchmark of the weight-streaming skinny GEMM on one MI355X.

One step = one pass of the hot path over one batch: the NVFP4 GEMMs of one
MLP block of a ~27B dense decoder at M=1 (gate_up 34816x5120 then down
5120x17408), every weight read from HBM in its packed form. Weights live in
enough distinct copies (>= 2 GiB) that no launch finds its matrix in the
256 MB last-level cache; inputs are resident in HBM before timing starts.

Prints one JSON line. ``value`` is the effective HBM read bandwidth of the
step (algorithmic bytes: packed codes + block scales + x + y, divided by the
step time); the timed steps follow at least SETTLE_MS of untimed replays of
the same step, back to back, so they run at settled clocks. Also reported:

* plain reads: the read-only kernel swept over grid x loads in flight for a
  4 GiB buffer (the measured ceiling), for one launch the size of the whole
  step, for each timed matrix's size, and for the step's two matrices as two
  back-to-back launches (the launch-for-launch floor of the step);
* per-matrix times for every workload (NVFP4 M=1, 8, 16; FP8 M=1, 2, 4, 8;
  the GEMV case; the per-GPU shapes of 4-way tensor parallelism; the output
  head, plain and with the greedy argmax), each against the same-size read;
* the full 64-layer decode step as stream-ordered launches and as one graph;
* the roofline of the dominant kernel;
* the CPU oracle (cpu_baseline leg): timed on sampled rows of every timed
  configuration (dequantize + matmul, and matmul alone), and used there to
  check the GPU's outputs for the same rows and activations.

``--quick`` keeps only the reads of the step's sizes and the headline step.
"""

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "effective HBM read GB/s (% of ceiling), NVFP4/FP8 skinny GEMM at M=1 and M=8"
PEAK_HBM_GBPS = 8000.0
ROTATE_BYTES = 2.5e9
MAX_COPIES = 256  # the GEMV case stays cache-resident even so (it is reported, not judged)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class mark:
    """A named ROCTx range around a measurement, so that a profiler run with
    marker tracing can attribute each kernel dispatch to its workload; a
    no-op when the ROCTx library is not there."""
    _lib = None

    def __init__(self, name):
        self.name = name.encode() if name else None
        if mark._lib is None:
            import ctypes
            mark._lib = False
            for so in ("librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"):
                try:
                    mark._lib = ctypes.CDLL(so)
                    break
                except OSError:
                    continue

    def __enter__(self):
        if mark._lib and self.name:
            mark._lib.roctxRangePushA(self.name)

    def __exit__(self, *exc):
        if mark._lib and self.name:
            mark._lib.roctxRangePop()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=1000)
    p.add_argument("--quick", action="store_true", help="only the headline step (for profiler runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--launches", default="",
                   help="profiling mode: comma-separated fmt:matrix:m[:full|ring|dot] cases (dot: the VALU "
                        "packed-dot path, full stage), each launched --steps times in order (after one warm-up "
                        "launch), then exit")
    return p.parse_args()


def run_launches(spec, steps):
    """Launch each case of `spec` `steps` times, stream-ordered, over enough
    rotating copies that no launch finds its weights in the last-level cache;
    for counter runs, which attribute dispatches by their order."""
    import torch
    import quantized_weight_skinny_amd as q
    from quantized_weight_skinny_amd import torch_api as qt
    stages = {"": 0, "full": q.QPN_X_STAGE_FULL, "ring": q.QPN_X_STAGE_RING, "dot": q.QPN_X_STAGE_FULL}
    done = []
    for case in spec.split(","):
        fmt, name, m, *rest = case.split(":")
        m, stage = int(m), stages[rest[0] if rest else ""]
        dot = int(bool(rest) and rest[0] == "dot")
        n, k = workloads.SHAPES[name]
        nbytes = q.qpn_packed_bytes(q.QPN_FMT_NVFP4 if fmt == "nvfp4" else q.QPN_FMT_FP8_E4M3, n, k)
        mat = Mat(name, fmt, "launches", copies=max(2, int(np.ceil(300e6 / nbytes))))
        x = torch.randn((m, mat.k), device="cuda").half()
        y = torch.empty((m, mat.n), dtype=torch.float16, device="cuda")
        ws = qt.new_workspace(mat.copies[0], m, x_stage=stage, valu_dot=dot)
        plan = q.qpn_gemm_plan(mat.copies[0].desc(), m, q.make_launch(x_stage=stage, valu_dot=dot))
        for i in range(steps + 1):
            qt.gemm(x, mat.copies[i % len(mat.copies)], out=y, workspace=ws, x_stage=stage, valu_dot=dot)
        torch.cuda.synchronize()
        done.append({"case": case, "dispatches": steps + 1, "split_k": plan.split_k, "waves": plan.waves_per_group,
                     "k_slices": plan.k_slices, "depth": plan.depth, "x_stage": plan.x_stage,
                     "whole_groups": plan.whole_groups, "valu_dot": plan.valu_dot})
        log(f"{case}: {steps + 1} launches, plan {done[-1]}")
        del mat
        torch.cuda.empty_cache()
    print(json.dumps({"launches": done}))


class Mat:
    """One packed weight in R rotating device copies."""

    def __init__(self, name, fmt, wl, copies=None):
        import torch
        from quantized_weight_skinny_amd import torch_api as qt
        self.name, self.fmt = name, fmt
        n, k = workloads.SHAPES[name]
        self.n, self.k = n, k
        self.wl = wl
        w = workloads.weights(n, k, workloads.seed_for(wl, name, "W"))
        # host copies the cpu_baseline leg needs: the sampled rows and the
        # tensor-wide amax (a plain max of the generated input)
        self.sample = sample_rows(n)
        self.w_rows = np.ascontiguousarray(w[self.sample])
        self.amax = float(np.abs(w).max())
        wd = torch.from_numpy(w).to("cuda")
        del w
        if fmt == "nvfp4":
            codes, scales, s_t = qt.quantize_nvfp4(wd)
            pw = qt.pack_nvfp4(codes, scales, s_t, n, k)
            del codes, scales
        else:
            codes, rs = qt.quantize_fp8(wd)
            pw = qt.pack_fp8(codes, rs, n, k)
            del codes
        del wd
        self.weight_bytes = pw.nbytes
        r = copies or min(MAX_COPIES, max(1, int(np.ceil(ROTATE_BYTES / self.weight_bytes))))
        self.copies = [pw]
        for _ in range(r - 1):
            rs = pw.row_scales.clone() if pw.row_scales is not None else None
            self.copies.append(qt.PackedWeight(pw.fmt, n, k, pw.packed.clone(), pw.tensor_scale, rs))
        torch.cuda.synchronize()

    def bytes_for(self, m, swiglu=False, argmax=False):
        out = 8 * m if argmax else 2 * m * (self.n // 2 if swiglu else self.n)
        return self.weight_bytes + 2 * m * self.k + out


def sample_rows(n):
    """Output rows the bench checks per configuration: the first and last 64,
    128 spread over N and 64 in the last eighth (where a balanced launch puts
    its split-K tail groups)."""
    rows = set(range(min(64, n))) | set(range(max(0, n - 64), n))
    rows |= set(np.linspace(0, n - 1, 128).astype(int).tolist())
    rows |= set(np.linspace(n - n // 8, n - 1, 64).astype(int).tolist())
    return np.array(sorted(rows), dtype=np.int64)


CHECKS = []


def gpu_sample(mat, m, label):
    """One launch of the timed plan on seeded activations; the sampled output
    columns are kept for the cpu_baseline leg, which computes the same rows
    with the oracle and compares (outside every timed region)."""
    import torch
    from quantized_weight_skinny_amd import torch_api as qt
    x = workloads.activations(m, mat.k, workloads.seed_for(mat.wl, mat.name, f"x{m}"))
    y = qt.gemm(torch.from_numpy(x).to("cuda"), mat.copies[0])
    torch.cuda.synchronize()
    CHECKS.append({"label": label, "fmt": mat.fmt, "name": mat.name, "n": mat.n, "k": mat.k, "m": m,
                   "rows": mat.sample, "w_rows": mat.w_rows, "amax": mat.amax, "x": x,
                   "y": y.cpu().numpy()[:, mat.sample].astype(np.float64)})


def capture(launches):
    """One HIP graph (torch.cuda.CUDAGraph) holding the given launch closures
    in order; outputs and workspaces are allocated before capture and the
    captured launches contain no memset."""
    import torch
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in launches:
            fn()
    torch.cuda.synchronize()
    return g


# Sustained streaming first: MI355X's clocks dip for about ten milliseconds
# after a streaming load starts and then settle (a graph of gate_up launches
# at M=1 goes 18.3 -> 23 -> 18.1 µs per launch over its first 25 replays, and
# again after a second of idle), so every measurement below is preceded by at
# least this much untimed work of the same kind, enqueued back to back with
# the timed part.
SETTLE_MS = 30.0


def settle(run, min_ms=SETTLE_MS):
    """Enqueue run() (one unit of the work about to be measured) repeatedly,
    untimed, until about min_ms of GPU time; returns without synchronizing,
    so the timed work follows on the stream with no idle gap."""
    import torch
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    run()
    e1.record(s)
    torch.cuda.synchronize()
    once = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(int(np.ceil(min_ms / once))):
        run()


def replay_us(g, per_replay, trials, stat="median", label=None):
    """µs per launch over `trials` replays of graph g (per_replay launches
    each), after replays that settle the clocks, timed with events on the
    launch stream between replays: the median of the per-replay means, or
    (stat="mean") the mean over all. `label` names the timed replays as a
    ROCTx range."""
    import torch
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
    settle(g.replay)
    with mark(label):
        ev[0].record(s)
        for i in range(trials):
            g.replay()
            ev[i + 1].record(s)
        torch.cuda.synchronize()
    if stat == "mean":
        return ev[0].elapsed_time(ev[-1]) * 1e3 / (trials * per_replay)
    return float(np.median([ev[i].elapsed_time(ev[i + 1]) * 1e3 / per_replay for i in range(trials)]))


def time_matrix(mat, m, reps=10, label=None, swiglu=False, argmax=False, stat="median"):
    """µs per launch of one matrix: a graph of back-to-back launches over all
    rotating copies, replayed `reps` times with events on the launch stream
    (the median over replays, or stat="mean": the average launch).
    ``swiglu``: the gate_up GEMM with the SwiGLU epilogue (output n/2 wide);
    ``argmax``: the greedy-argmax epilogue (an index and a value per row)."""
    tag = "_swiglu" if swiglu else "_argmax" if argmax else ""
    return _time_matrix(mat, m, reps, swiglu, argmax, stat, label or f"{mat.fmt}_m{m}/{mat.name}{tag}")


def _time_matrix(mat, m, reps, swiglu=False, argmax=False, stat="median", label=None):
    import torch
    from quantized_weight_skinny_amd import torch_api as qt
    x = torch.randn((m, mat.k), device="cuda").half()
    y = torch.empty((m, mat.n // 2 if swiglu else mat.n), dtype=torch.float16, device="cuda")
    if argmax:
        ws = qt.argmax_workspace(mat.copies[0], m)
        idx = torch.empty(m, dtype=torch.int32, device="cuda")
        val = torch.empty(m, dtype=torch.float32, device="cuda")
        launches = [(lambda c=c: qt.gemm_argmax(x, c, idx=idx, val=val, workspace=ws)) for c in mat.copies]
    else:
        ws = qt.new_workspace(mat.copies[0], m, swiglu=swiglu)
        run = qt.gemm_swiglu if swiglu else qt.gemm
        launches = [(lambda c=c: run(x, c, out=y, workspace=ws)) for c in mat.copies]
    for fn in launches:
        fn()
    g = capture(launches)
    g.replay()
    torch.cuda.synchronize()
    us = replay_us(g, len(launches), reps, stat, label)
    del g
    return us, mat.bytes_for(m, swiglu, argmax) / (us * 1e-6) / 1e9


def time_mlp(gate_up, down, m, reps=10, one_launch=False):
    """The MLP of one layer as the decoder runs it: x -> gate_up with the
    SwiGLU epilogue -> h -> down -> y, over the rotating copies, one graph:
    as two GEMM launches, or (one_launch) as qpn_mlp's one-launch form.
    Returns (µs per MLP, GB/s over weights + x + h written and read + y)."""
    import torch
    from quantized_weight_skinny_amd import torch_api as qt
    x = torch.randn((m, gate_up.k), device="cuda").half()
    h = torch.empty((m, gate_up.n // 2), dtype=torch.float16, device="cuda")
    y = torch.empty((m, down.n), dtype=torch.float16, device="cuda")
    ws_g = qt.new_workspace(gate_up.copies[0], m, swiglu=True)
    ws_d = qt.new_workspace(down.copies[0], m)
    ws_f = qt.mlp_workspace(gate_up.copies[0], down.copies[0], m, fused=1) if one_launch else None
    r = min(len(gate_up.copies), len(down.copies))

    def mlp(i):
        if one_launch:
            qt.mlp(x, gate_up.copies[i], down.copies[i], h=h, y=y, workspace=ws_f, fused=1)
            return
        qt.gemm_swiglu(x, gate_up.copies[i], out=h, workspace=ws_g)
        qt.gemm(h, down.copies[i], out=y, workspace=ws_d)

    for i in range(r):
        mlp(i)
    g = capture([(lambda i=i: mlp(i)) for i in range(r)])
    g.replay()
    torch.cuda.synchronize()
    us = replay_us(g, r, reps, label=f"nvfp4_m{m}/mlp_{'one_launch' if one_launch else 'swiglu'}")
    del g
    nbytes = gate_up.bytes_for(m, swiglu=True) + down.bytes_for(m)
    return us, nbytes / (us * 1e-6) / 1e9


READ_GRIDS = (256, 512, 768, 1024, 1536, 2048, 3072, 4096)
READ_LOADS = (2, 4, 8)


def _read_graph_us(buf, size, grid, loads, reps):
    """µs per launch of the read kernel over `size`-byte slices of `buf`
    (rotating, a graph of back-to-back launches), settled clocks, median of
    `reps` replays."""
    import torch
    from quantized_weight_skinny_amd import torch_api as qt
    nsl = max(1, min(64, buf.numel() // size))
    slices = [buf[i * size:(i + 1) * size] for i in range(nsl)]
    sink = torch.empty(grid * 4, dtype=torch.int32, device="cuda")
    launches = [(lambda sl=sl: qt.read_ceiling(sl, grid, sink, loads)) for sl in slices]
    for fn in launches:
        fn()
    g = capture(launches)
    us = replay_us(g, len(launches), reps)
    del g
    return us


def read_sweep(sizes, total=4 << 30, reps=5):
    """The best plain read a single launch of each size can make: the read
    kernel over rotating slices of a `total`-byte buffer, swept over
    READ_GRIDS x READ_LOADS (loads in flight per thread), settled clocks.
    Returns {name: {"bytes", "us", "GBps", "grid", "loads"}} (GB/s = bytes per
    launch / µs per launch, the launch gap of a graph replay included)."""
    import torch
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    out = {}
    for name, nbytes in sizes.items():
        size = min(total, (int(nbytes) + 255) // 256 * 256)
        best = None
        for grid in READ_GRIDS:
            for loads in READ_LOADS:
                us = _read_graph_us(buf, size, grid, loads, reps)
                if best is None or us < best[0]:
                    best = (us, grid, loads)
        out[name] = {"bytes": size, "us": round(best[0], 3), "GBps": round(size / (best[0] * 1e-6) / 1e9, 1),
                     "grid": best[1], "loads": best[2]}
        log(f"read {name} ({size / 1e6:.1f} MB): {best[0]:.2f} us, {out[name]['GBps']:.0f} GB/s "
            f"(grid {best[1]}, {best[2]} loads)")
    del buf
    torch.cuda.empty_cache()
    return out


def read_pair_us(a, b, total=4 << 30, reps=5):
    """µs per pair of back-to-back plain reads of the sizes and launch shapes
    a and b (two entries of read_sweep): the launch-for-launch floor of a
    two-GEMM step."""
    import torch
    from quantized_weight_skinny_amd import torch_api as qt
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    span = a["bytes"] + b["bytes"]
    npair = max(1, min(32, total // span))
    sink = torch.empty(4096 * 4, dtype=torch.int32, device="cuda")
    launches = []
    for i in range(npair):
        base = i * span
        sa, sb = buf[base:base + a["bytes"]], buf[base + a["bytes"]:base + span]
        launches.append(lambda sa=sa, sb=sb: (qt.read_ceiling(sa, a["grid"], sink, a["loads"]),
                                              qt.read_ceiling(sb, b["grid"], sink, b["loads"])))
    for fn in launches:
        fn()
    g = capture(launches)
    us = replay_us(g, len(launches), reps)
    del g, buf
    torch.cuda.empty_cache()
    return us


KERNEL_SOURCES = ("qpn_device.hpp", "qpn_gemm.hip", "qpn_gemm_body.hpp", "qpn_internal.hpp", "qpn_plan.hpp",
                  "qpn_plan.cpp")


def kernel_source_hash():
    """sha256 over the sources that define the GEMM kernel and its launch
    plan (the C-ABI wrapper and the offline kernels do not enter it)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_weight_skinny_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_nvfp4_gate_up_m1_traffic.md")


def kernel_traffic():
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, or None when the kernel sources changed after
    the counters were taken (the summary records the source hash)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def decode_step(ms=(1, 2, 4, 8), reps=3):
    """The synthetic decode step of a ~27B dense decoder: 64 layers of
    [qkv FP8, o_proj FP8, gate_up NVFP4, down NVFP4], then the NVFP4 lm_head,
    each layer's weights at their own addresses (14.1 GB in all), launched in
    order, once from the host one launch at a time and once as one HIP graph.
    Returns {m: (graph ms per step, graph GB/s, bytes, stream-ordered ms)}."""
    import torch
    from quantized_weight_skinny_amd import torch_api as qt
    wl = "decode_step_27b"
    protos = {}
    for name, fmt in workloads.DECODE_LAYER_MATS:
        protos[name] = Mat(name, fmt, wl, copies=workloads.DECODE_LAYERS)
    head = Mat("lm_head", "nvfp4", wl, copies=1)
    out = {}
    for m in ms:
        launches, total = [], 0
        bufs = {}
        for name, _ in workloads.DECODE_LAYER_MATS + (("lm_head", "nvfp4"),):
            n, k = workloads.SHAPES[name]
            mat = head if name == "lm_head" else protos[name]
            bufs[name] = (torch.randn((m, k), device="cuda").half(),
                          torch.empty((m, n), dtype=torch.float16, device="cuda"),
                          qt.new_workspace(mat.copies[0], m))
        for layer in range(workloads.DECODE_LAYERS):
            for name, _ in workloads.DECODE_LAYER_MATS:
                x, y, ws = bufs[name]
                c = protos[name].copies[layer]
                launches.append(lambda x=x, c=c, y=y, ws=ws: qt.gemm(x, c, out=y, workspace=ws))
                total += protos[name].bytes_for(m)
        x, y, ws = bufs["lm_head"]
        launches.append(lambda x=x, c=head.copies[0], y=y, ws=ws: qt.gemm(x, c, out=y, workspace=ws))
        total += head.bytes_for(m)
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # stream-ordered: the launches issued one by one from the host
        for fn in launches:
            fn()
        torch.cuda.synchronize()

        def one_step():
            for fn in launches:
                fn()

        settle(one_step)
        with mark(f"decode_m{m}/stream"):
            e0.record(s)
            for _ in range(reps):
                for fn in launches:
                    fn()
            e1.record(s)
            torch.cuda.synchronize()
        ms_stream = e0.elapsed_time(e1) / reps
        # one HIP graph holding the whole step
        g = capture(launches)
        g.replay()
        torch.cuda.synchronize()
        settle(g.replay)
        with mark(f"decode_m{m}/graph"):
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
            torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / reps
        out[m] = (ms_step, total / (ms_step * 1e-3) / 1e9, total, ms_stream)
        log(f"decode step M={m}: graph {ms_step:.3f} ms, {out[m][1]:.0f} GB/s; stream-ordered {ms_stream:.3f} ms, "
            f"{total / (ms_stream * 1e-3) / 1e9:.0f} GB/s; {total / 1e9:.2f} GB, {len(launches)} GEMMs")
        del g
    del protos, head
    torch.cuda.empty_cache()
    return out


def cpu_baseline(min_s=0.3):
    """The oracle as it stands (numpy: float64 dequantize, then float64
    matmul) on the bench's sampled rows of every timed configuration: the
    oracle quantizes the sampled rows of W itself (untimed; NVFP4 with the
    tensor scale of the whole matrix's amax), then dequantize + matmul and
    matmul alone are timed (repeated for at least ``min_s`` each), and the
    GPU's outputs for the same rows and activations are checked against the
    result (|y_gpu - y| <= 2e-3 sum|wx| + 1e-3). GB/s count the sample's
    algorithmic bytes. The 64-layer decode step at M=1 is composed from the
    per-matrix rates (64 x per layer + lm_head)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    rows_out, checks_ok = [], True
    rate = {}
    for c in CHECKS:
        w, m, n, k = c["w_rows"], c["m"], c["n"], c["k"]
        r = len(c["rows"])
        if c["fmt"] == "nvfp4":
            codes, sc, s_t = oracle.quantize_nvfp4(w, oracle.nvfp4_tensor_scale(c["amax"]))
            row_bytes = k // 2 + k // 16
            deq = lambda: oracle.dequantize_nvfp4(codes, sc, s_t)  # noqa: E731
        else:
            codes, rs = oracle.quantize_fp8(w)
            row_bytes = k + 4
            deq = lambda: oracle.dequantize_fp8(codes, rs)  # noqa: E731
        x = c["x"].astype(np.float64)
        t0, reps = time.perf_counter(), 0
        while True:
            wdq = deq()
            y_ref = x @ wdq.T
            reps += 1
            if time.perf_counter() - t0 >= min_s:
                break
        t_total = (time.perf_counter() - t0) / reps
        t0, reps2 = time.perf_counter(), 0
        while True:
            y_ref = x @ wdq.T
            reps2 += 1
            if time.perf_counter() - t0 >= min_s:
                break
        t_mm = (time.perf_counter() - t0) / reps2
        b = np.abs(x) @ np.abs(wdq).T
        tol = 2e-3 * b + 1e-3
        excess = float(np.max(np.abs(c["y"] - y_ref) / tol))
        ok = bool(excess <= 1.0)
        checks_ok &= ok
        nbytes = r * row_bytes + 2 * m * k + 2 * m * r
        per_row_s = t_total / r
        rate[(c["fmt"], c["name"], m)] = (per_row_s, row_bytes)
        rows_out.append({"config": c["label"], "rows": r, "total_s": round(t_total, 5), "matmul_s": round(t_mm, 6),
                         "GBps": round(nbytes / t_total / 1e9, 4), "matmul_only_GBps": round(nbytes / t_mm / 1e9, 4),
                         "gpu_check": "pass" if ok else "FAIL", "max_err_over_bound": round(excess, 4)})
        log(f"cpu {c['label']}: {r} rows, {nbytes / t_total / 1e9:.3f} GB/s (matmul only {nbytes / t_mm / 1e9:.2f}); "
            f"gpu check {'pass' if ok else 'FAIL'} (max err / bound {excess:.3f})")
    # the headline workload (gate_up + down at M = 1) as one rate
    head = [row for row in rows_out if row["config"] in ("nvfp4_m1/gate_up", "nvfp4_m1/down")]
    value = None
    if head:
        tot_b = sum(row["GBps"] * row["total_s"] * 1e9 for row in head)
        value = tot_b / sum(row["total_s"] for row in head) / 1e9
    composed = None
    need = [("fp8", "qkv", 1), ("fp8", "o_proj", 1), ("nvfp4", "gate_up", 1), ("nvfp4", "down", 1),
            ("nvfp4", "lm_head", 1)]
    if all(key in rate for key in need):
        t_layer = sum(rate[key][0] * workloads.SHAPES[key[1]][0] for key in need[:4])
        t_head = rate[need[4]][0] * workloads.SHAPES["lm_head"][0]
        t_step = workloads.DECODE_LAYERS * t_layer + t_head
        step_bytes = sum(rate[key][1] * workloads.SHAPES[key[1]][0] for key in need[:4]) * workloads.DECODE_LAYERS \
            + rate[need[4]][1] * workloads.SHAPES["lm_head"][0]
        composed = {"m": 1, "s_per_step": round(t_step, 3), "weight_GBps": round(step_bytes / t_step / 1e9, 4),
                    "kind": "composed: 64 x (qkv FP8 + o_proj FP8 + gate_up NVFP4 + down NVFP4) + lm_head NVFP4, "
                            "each from its sampled-row rate scaled to all rows"}
    return {"value": round(value, 4) if value is not None else None, "unit": "GB/s", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"{len(CHECKS)} configurations, the bench's sampled output rows of each (first/last 64, 128 "
                      "spread, 64 in the last eighth of N), all M activation rows; numpy float64 dequantize + matmul; "
                      "value = gate_up + down at M=1",
            "gpu_checks": "pass" if checks_ok else "FAIL", "rows": rows_out, "decode_step_27b_composed": composed}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the library has no collective "
                                   "(the all-reduce of a row-parallel layer), so --gpus > 1 is refused",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    import quantized_weight_skinny_amd as q
    from quantized_weight_skinny_amd import torch_api as qt  # noqa: F401  (fails loudly without libqpn.so)
    if args.launches:
        run_launches(args.launches, args.steps)
        return

    nv = lambda name: q.qpn_packed_bytes(q.QPN_FMT_NVFP4, *workloads.SHAPES[name])  # noqa: E731
    f8 = lambda name: q.qpn_packed_bytes(q.QPN_FMT_FP8_E4M3, *workloads.SHAPES[name]) + 4 * workloads.SHAPES[name][0]  # noqa: E731,E501
    sizes = {"ceiling_4GiB": 4 << 30, "step": nv("gate_up") + nv("down"), "gate_up": nv("gate_up"), "down": nv("down")}
    if not args.quick:
        sizes.update({"qkv_nvfp4": nv("qkv"), "o_proj_nvfp4": nv("o_proj"), "qkv_fp8": f8("qkv"),
                      "o_proj_fp8": f8("o_proj"), "down_fp8": f8("down"), "lm_head": nv("lm_head")})
    log("plain reads (grid x loads sweep per size)")
    with mark("read_sweep"):
        reads = read_sweep(sizes)
    ceiling = reads["ceiling_4GiB"]["GBps"]
    pair_us = read_pair_us(reads["gate_up"], reads["down"])
    log(f"ceiling {ceiling:.0f} GB/s; gate_up + down as two plain reads: {pair_us:.2f} us a pair")

    log("building rotating weights for the M=1 MLP step")
    wl = "nvfp4_27b_m1"
    gate_up = Mat("gate_up", "nvfp4", wl)
    r_steps = len(gate_up.copies)
    down = Mat("down", "nvfp4", wl, copies=r_steps)
    m = 1
    x1 = torch.randn((m, 5120), device="cuda").half()
    x2 = torch.randn((m, 17408), device="cuda").half()
    h = torch.empty((m, 34816), dtype=torch.float16, device="cuda")
    y = torch.empty((m, 5120), dtype=torch.float16, device="cuda")
    ws_g = qt.new_workspace(gate_up.copies[0], m)
    ws_d = qt.new_workspace(down.copies[0], m)
    step_bytes = gate_up.bytes_for(m) + down.bytes_for(m)
    gate_up_bytes = gate_up.bytes_for(m)

    def step(i):
        qt.gemm(x1, gate_up.copies[i % r_steps], out=h, workspace=ws_g)
        qt.gemm(x2, down.copies[i % r_steps], out=y, workspace=ws_d)

    # One HIP graph holds one cycle of steps (every rotating copy once); the W
    # warmup steps, the settling replays and the K timed steps are replays of
    # it, plus a graph of the leftover steps when W or K is not a whole number
    # of cycles. The cycle graph is checked against the eager step first.
    for i in range(r_steps):
        step(i)
    torch.cuda.synchronize()
    eager_y = y.clone()
    cycle = capture([(lambda i=i: step(i)) for i in range(r_steps)])
    leftover = {n % r_steps: capture([(lambda i=i: step(i)) for i in range(n % r_steps)])
                for n in (args.warmup, args.steps) if n % r_steps}
    cycle.replay()
    torch.cuda.synchronize()
    if not torch.equal(y, eager_y):
        raise SystemExit("graph replay does not reproduce the eager step")

    def run_steps(n):
        for _ in range(n // r_steps):
            cycle.replay()
        if n % r_steps:
            leftover[n % r_steps].replay()

    s = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with mark("step/warmup"):
        run_steps(args.warmup)
    torch.cuda.synchronize()
    # After the synchronize the GPU is idle, and an idle GPU restarts the
    # clock transient of a streaming load; untimed replays of the same step
    # (at least SETTLE_MS of GPU time) run back to back before the timed ones,
    # so the timed steps see the same settled clocks as every other row.
    settle_t0 = time.perf_counter()
    settle(cycle.replay)
    wall0 = time.perf_counter()
    with mark("step/timed"):
        t0.record(s)
        run_steps(args.steps)
        t1.record(s)
        torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9
    del cycle, leftover
    log(f"settle enqueued in {1e3 * (wall0 - settle_t0):.1f} ms of host time")

    # The dominant kernel (gate_up): a graph of back-to-back launches over
    # the rotating copies, events on the launch stream around it.
    gate_up_us, achieved = time_matrix(gate_up, m, reps=10, label="roofline/nvfp4_m1/gate_up", stat="mean")
    traffic = kernel_traffic()
    log(f"step {ms_step * 1e3:.1f} us, {value:.0f} GB/s; gate_up {gate_up_us:.1f} us per launch, "
        f"{achieved:.0f} GB/s; wall {wall:.3f} s; traffic {traffic}")

    extras = {}
    decode = None
    same_size = {"gate_up": "gate_up", "gate_up_swiglu": "gate_up", "down": "down"}
    if not args.quick:
        per = {}
        for mm in (1, 8, 16):
            per[f"nvfp4_m{mm}/gate_up"] = time_matrix(gate_up, mm)
            gpu_sample(gate_up, mm, f"nvfp4_m{mm}/gate_up")
            per[f"nvfp4_m{mm}/down"] = time_matrix(down, mm)
            gpu_sample(down, mm, f"nvfp4_m{mm}/down")
        for mm in (1, 8):
            per[f"nvfp4_m{mm}/gate_up_swiglu"] = time_matrix(gate_up, mm, swiglu=True)
            per[f"nvfp4_m{mm}/mlp_swiglu"] = time_mlp(gate_up, down, mm)
        # qpn_mlp's one-launch form (on request only: level with the two
        # launches at one and two rows), with the two-launch form at two rows
        # beside it
        per["nvfp4_m1/mlp_one_launch"] = time_mlp(gate_up, down, 1, one_launch=True)
        per["nvfp4_m2/mlp_swiglu"] = time_mlp(gate_up, down, 2)
        per["nvfp4_m2/mlp_one_launch"] = time_mlp(gate_up, down, 2, one_launch=True)
        del gate_up, down
        torch.cuda.empty_cache()
        for name in ("qkv", "o_proj"):
            mat = Mat(name, "nvfp4", "nvfp4_27b_m8")
            for mm in (1, 8):
                per[f"nvfp4_m{mm}/{name}"] = time_matrix(mat, mm)
                gpu_sample(mat, mm, f"nvfp4_m{mm}/{name}")
            del mat
            torch.cuda.empty_cache()
        for name in ("qkv", "down", "o_proj"):
            mat = Mat(name, "fp8", "fp8_27b_m124")
            for mm in (1, 2, 4, 8):
                per[f"fp8_m{mm}/{name}"] = time_matrix(mat, mm)
                gpu_sample(mat, mm, f"fp8_m{mm}/{name}")
            del mat
            torch.cuda.empty_cache()
        mat = Mat("gemv", "nvfp4", "nvfp4_gemv_m1")
        per["nvfp4_m1/gemv"] = time_matrix(mat, 1)
        gpu_sample(mat, 1, "nvfp4_m1/gemv")
        del mat
        for name in ("qkv_tp4", "o_proj_tp4", "gate_up_tp4", "down_tp4"):
            mat = Mat(name, "nvfp4", "nvfp4_27b_tp4")
            for mm in (1, 8):
                per[f"nvfp4_m{mm}/{name}"] = time_matrix(mat, mm)
                gpu_sample(mat, mm, f"nvfp4_m{mm}/{name}")
            del mat
            torch.cuda.empty_cache()
        head = Mat("lm_head", "nvfp4", "decode_step_27b", copies=6)
        for mm in (1, 8):
            per[f"nvfp4_m{mm}/lm_head"] = time_matrix(head, mm)
            gpu_sample(head, mm, f"nvfp4_m{mm}/lm_head")
            per[f"nvfp4_m{mm}/lm_head_argmax"] = time_matrix(head, mm, argmax=True)
        del head
        torch.cuda.empty_cache()
        same_size.update({"qkv": "qkv_nvfp4", "o_proj": "o_proj_nvfp4", "lm_head": "lm_head",
                          "lm_head_argmax": "lm_head"})
        same_size_f8 = {"qkv": "qkv_fp8", "o_proj": "o_proj_fp8", "down": "down_fp8"}
        for key, (us, gbps) in per.items():
            row = {"us": round(us, 2), "GBps": round(gbps, 1), "frac_of_measured_ceiling": round(gbps / ceiling, 4)}
            fmt_m, name = key.split("/")
            ref = (same_size_f8 if fmt_m.startswith("fp8") else same_size).get(name)
            if ref in reads:
                row["same_size_read_us"] = reads[ref]["us"]
                row["frac_of_same_size_read"] = round(reads[ref]["us"] / us, 4)
            extras[key] = row
            log(f"{key}: {us:.1f} us {gbps:.0f} GB/s ({100 * gbps / ceiling:.1f}% of ceiling)")
        decode = {str(m): {"ms_per_step": round(v[0], 4), "GBps": round(v[1], 1),
                           "weight_and_io_bytes": v[2], "frac_of_measured_ceiling": round(v[1] / ceiling, 4),
                           "stream_ordered_ms_per_step": round(v[3], 4),
                           "stream_ordered_GBps": round(v[2] / (v[3] * 1e-3) / 1e9, 1)}
                  for m, v in decode_step().items()}

    cpu = None
    if not args.no_cpu_baseline:
        if not CHECKS:
            gate_up = Mat("gate_up", "nvfp4", wl, copies=1)
            gpu_sample(gate_up, 1, "nvfp4_m1/gate_up")
            del gate_up
            down = Mat("down", "nvfp4", wl, copies=1)
            gpu_sample(down, 1, "nvfp4_m1/down")
            del down
        log("cpu baseline (oracle) and the check of every timed configuration")
        cpu = cpu_baseline()
        log(f"cpu baseline {cpu['value']} GB/s; gpu checks {cpu['gpu_checks']}")

    try:
        sha = subprocess.run(["git", "rev-parse", "--short", "HEAD"], capture_output=True, text=True,
                             cwd=ROOT).stdout.strip() or None
    except Exception:
        sha = None
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "nvfp4_27b_m1: NVFP4 gate_up 34816x5120 + down 5120x17408, M=1",
                   "m": 1, "format": "nvfp4", "rotating_copies": r_steps, "step_bytes": step_bytes,
                   "settle_ms": SETTLE_MS},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "kernel": "gemm_kernel<NVFP4> on gate_up 34816x5120, M=1",
                     "launch_us": round(gate_up_us, 3), "algorithmic_bytes": gate_up_bytes},
        "measured_read_ceiling_GBps": ceiling,
        "frac_of_measured_ceiling": round(value / ceiling, 4),
        "plain_reads": reads,
        "step_as_two_plain_reads_us": round(pair_us, 3),
        "frac_of_two_plain_reads": round(pair_us / (ms_step * 1e3), 4),
        "frac_of_step_sized_read": round(reads["step"]["us"] / (ms_step * 1e3), 4),
        "cpu_baseline": cpu,
        "per_matrix": extras,
        "decode_step_27b": decode,
        "git": sha,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
