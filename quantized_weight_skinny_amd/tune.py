"""Launch-shape tuner: the fastest qpn_gemm_tuned launch for one GEMM shape.

For a weight format, an [n, k] shape and m activation rows, the tuner sweeps
the launch shapes the planner accepts (wavefronts per workgroup, K slices, K
split, groups kept whole, stream depth, activation stage) on synthetic
weights, then times the best few and the planner's current choice again in
alternated rounds, and prints the winner as an entry of the planner's launch
table (``kTuned`` in ``csrc/qpn_plan.cpp``).

Each timing is a HIP graph of back-to-back launches over rotating copies of
the weight (at least 2.5 GB in all, so that no launch finds its weights in a
cache; at most 256 copies), replayed after 30 ms of untimed replays
of the same graph (the clocks settle), as the median over replays of the time
per launch.

    python -m quantized_weight_skinny_amd.tune --fmt nvfp4 --n 34816 --k 5120 --m 1

Outputs are not checked here (the GPU tests cover every launch shape); the
tuner only times.
"""

import argparse
import itertools
import statistics
import sys

from . import (
    QPN_FMT_FP8_E4M3,
    QPN_FMT_NVFP4,
    QPN_X_STAGE_FULL,
    QPN_X_STAGE_RING,
    QpnError,
    make_launch,
    make_weight,
    qpn_gemm_plan,
)

SETTLE_MS = 30.0
ROTATE_BYTES = 2_500_000_000  # as the benchmark: well past the memory-side cache
MAX_COPIES = 256  # small weights rotate through at most this many copies
FIELDS = ("waves", "k_slices", "split_k", "depth", "x_stage", "whole_groups")
UNEVEN_WAVES = 9  # workgroup size of the planner's uneven-group grid


def planner_weight(fmt, n, k):
    """A weight descriptor for plan queries (the planner reads no memory)."""
    return make_weight(fmt, n, k, 1 << 20, 1.0, (1 << 20) if fmt == QPN_FMT_FP8_E4M3 else None)


def current_plan(fmt, n, k, m):
    """The launch the planner picks for this shape today, as a dict."""
    p = qpn_gemm_plan(planner_weight(fmt, n, k), m)
    return dict(waves=p.waves_per_group, k_slices=p.k_slices, split_k=p.split_k, depth=p.depth,
                x_stage=p.x_stage, whole_groups=p.whole_groups)


def candidates(fmt, n, k, m, cus):
    """Every launch shape of the sweep grid that the planner accepts for this
    shape, resolved (so that equal launches appear once). With a K split, the
    groups are either all split or, where there are more groups than CUs, the
    leading multiple of the CU count is kept whole (a balanced grid). For
    NVFP4 the uneven grid of one workgroup per CU (UNEVEN_WAVES wavefronts)
    joins in where the planner takes it."""
    w = planner_weight(fmt, n, k)
    seen, out = set(), []

    def add(launch):
        try:
            p = qpn_gemm_plan(w, m, launch)
        except QpnError:
            return
        kw = dict(waves=p.waves_per_group, k_slices=p.k_slices, split_k=p.split_k, depth=p.depth,
                  x_stage=p.x_stage, whole_groups=p.whole_groups)
        key = tuple(kw[f] for f in FIELDS)
        if key not in seen:
            seen.add(key)
            out.append(kw)

    for waves, ks, split, depth, stage in itertools.product(
            (4, 8), (1, 2, 4, 8), (1, 2, 3, 4, 6), (2, 3, 4), (QPN_X_STAGE_FULL, QPN_X_STAGE_RING)):
        if ks > waves:
            continue
        n_tiles = -(-n // 16)
        groups = -(-n_tiles // (waves // ks))
        wholes = [0]
        if split > 1 and groups > cus:
            wholes.append(groups // cus * cus)
        for whole in wholes:
            add(make_launch(split, waves, depth, ks, x_stage=stage, whole_groups=whole))
    for depth, stage in itertools.product((2, 3), (QPN_X_STAGE_FULL, QPN_X_STAGE_RING)):
        add(make_launch(1, UNEVEN_WAVES, depth, 1, x_stage=stage, whole_groups=cus))
    return out


def table_entry(fmt, n, k, m_max, kw):
    """A kTuned line for this launch."""
    stage = "kStageRing" if kw["x_stage"] == QPN_X_STAGE_RING else "kStageFull"
    f = "kFmtNvfp4" if fmt == QPN_FMT_NVFP4 else "kFmtFp8"
    waves = "kUnevenWaves" if kw["waves"] == UNEVEN_WAVES else kw["waves"]
    return (f"{{{f}, {n}, {k}, {m_max}, {waves}, {kw['k_slices']}, {kw['split_k']}, {kw['depth']}, {stage}, "
            f"{kw['whole_groups']}}}")


class Bench:
    """Synthetic weights in rotating copies, and the graph timing of one launch shape."""

    def __init__(self, fmt, n, k, seed=1234):
        import torch
        from . import torch_api as qt
        self.torch, self.qt = torch, qt
        self.fmt, self.n, self.k = fmt, n, k
        g = torch.Generator(device="cuda").manual_seed(seed)
        w = torch.randn((n, k), generator=g, device="cuda") * 0.02
        if fmt == QPN_FMT_NVFP4:
            codes, scales, s_t = qt.quantize_nvfp4(w)
            pw = qt.pack_nvfp4(codes, scales, s_t, n, k)
        else:
            codes, rs = qt.quantize_fp8(w)
            pw = qt.pack_fp8(codes, rs, n, k)
        del w
        count = min(MAX_COPIES, max(1, -(-ROTATE_BYTES // pw.nbytes)))
        self.copies = [pw] + [qt.PackedWeight(pw.fmt, n, k, pw.packed.clone(), pw.tensor_scale,
                                              pw.row_scales.clone() if pw.row_scales is not None else None)
                              for _ in range(count - 1)]
        torch.cuda.synchronize()

    def time(self, m, kw, reps=8):
        """µs per launch: median over reps graph replays, after SETTLE_MS of untimed ones."""
        torch, qt = self.torch, self.qt
        x = torch.randn((m, self.k), device="cuda").half()
        y = torch.empty((m, self.n), dtype=torch.float16, device="cuda")
        ws = qt.new_workspace(self.copies[0], m, **kw)
        calls = [(lambda c=c: qt.gemm(x, c, out=y, workspace=ws, **kw)) for c in self.copies]
        for fn in calls:
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for fn in calls:
                fn()
        graph.replay()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        graph.replay()
        e1.record(s)
        torch.cuda.synchronize()
        once = max(e0.elapsed_time(e1), 1e-3)
        for _ in range(int(SETTLE_MS / once) + 1):
            graph.replay()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(s)
        for i in range(reps):
            graph.replay()
            ev[i + 1].record(s)
        torch.cuda.synchronize()
        return statistics.median(ev[i].elapsed_time(ev[i + 1]) * 1e3 / len(calls) for i in range(reps))


def tune(fmt, n, k, m, top=5, rounds=5, log=print):
    """Sweep, then alternated rounds of the best `top` and the current plan.
    Returns [(median µs, launch dict, is_current)] fastest first."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cands = candidates(fmt, n, k, m, cus)
    cur = current_plan(fmt, n, k, m)
    bench = Bench(fmt, n, k)
    log(f"{len(cands)} launch shapes; {len(bench.copies)} copies of {bench.copies[0].nbytes / 1e6:.1f} MB")
    first = sorted(((bench.time(m, kw, reps=4), i) for i, kw in enumerate(cands)), key=lambda t: t[0])
    finalists = [cands[i] for _, i in first[:top]]
    if cur not in finalists:
        finalists.append(cur)
    times = [[] for _ in finalists]
    for _ in range(rounds):
        for i, kw in enumerate(finalists):
            times[i].append(bench.time(m, kw))
    res = sorted(((statistics.median(t), kw, kw == cur) for t, kw in zip(times, finalists)), key=lambda r: r[0])
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--fmt", choices=("nvfp4", "fp8"), required=True)
    ap.add_argument("--n", type=int, required=True)
    ap.add_argument("--k", type=int, required=True)
    ap.add_argument("--m", type=int, required=True)
    ap.add_argument("--top", type=int, default=5, help="finalists timed again in alternated rounds")
    ap.add_argument("--rounds", type=int, default=5)
    a = ap.parse_args(argv)
    fmt = QPN_FMT_NVFP4 if a.fmt == "nvfp4" else QPN_FMT_FP8_E4M3
    log = lambda *s: print(*s, flush=True)  # noqa: E731
    res = tune(fmt, a.n, a.k, a.m, a.top, a.rounds, log)
    log(f"\n{a.fmt} [{a.n} x {a.k}], m = {a.m}: median µs per launch over {a.rounds} alternated rounds")
    log("| µs | waves | k_slices | split_k | depth | stage | whole_groups | |")
    log("|---|---|---|---|---|---|---|---|")
    for us, kw, is_cur in res:
        stage = "ring" if kw["x_stage"] == QPN_X_STAGE_RING else "full"
        log(f"| {us:.2f} | {kw['waves']} | {kw['k_slices']} | {kw['split_k']} | {kw['depth']} | {stage} | "
            f"{kw['whole_groups']} | {'current plan' if is_cur else ''} |")
    log(f"\nfastest as a table entry: {table_entry(fmt, a.n, a.k, a.m, res[0][1])}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
