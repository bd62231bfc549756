"""CPU checks of libqpn.so: it loads, exports every entry point of
include/qpn.h, and rejects bad arguments on the host before any HIP call
(so these run without a GPU; no compute entry point is exercised)."""

import ctypes
import os
import re
import subprocess

import pytest

import quantized_weight_skinny_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qpn.h")

FAKE = 0x7F0000000000  # an aligned non-null "device" address; never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qpn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = q.lib()
    declared = _declared_functions()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), name
        assert name in q.SIGNATURES, name
    assert set(q.SIGNATURES) == set(declared)


def test_header_compiles_as_c99_and_links(tmp_path):
    """A plain C99 program includes qpn.h, links against libqpn.so with every
    declared entry point taken by address, and sees the struct layouts the
    Python binding uses (host-only calls, no device work)."""
    src = os.path.join(ROOT, "tests", "c_consumer", "qpn_c_consumer.c")
    text = open(src).read()
    for name in _declared_functions():
        assert f"(entry_fn){name}," in text, name
    libdir = os.path.dirname(q.LIB_PATH)
    exe = str(tmp_path / "qpn_c_consumer")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), src,
           "-o", exe, "-L", libdir, "-lqpn", f"-Wl,-rpath,{libdir}"]
    if os.path.isdir("/opt/rocm/lib"):
        cmd.append("-Wl,-rpath-link,/opt/rocm/lib")
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    got = dict(line.split(" ", 1) for line in run.stdout.splitlines())
    assert got["ok"] == "1"
    assert int(got["entries"]) == len(_declared_functions())
    assert int(got["sizeof_weight"]) == ctypes.sizeof(q.qpn_weight)
    assert int(got["offset_weight_n"]) == q.qpn_weight.n.offset
    assert int(got["offset_weight_packed"]) == q.qpn_weight.packed.offset
    assert int(got["offset_weight_tensor_scale"]) == q.qpn_weight.tensor_scale.offset
    assert int(got["offset_weight_row_scales"]) == q.qpn_weight.row_scales.offset
    assert int(got["sizeof_launch"]) == ctypes.sizeof(q.qpn_launch)
    assert int(got["offset_launch_whole_groups"]) == q.qpn_launch.whole_groups.offset
    assert int(got["offset_launch_block_columns"]) == q.qpn_launch.block_columns.offset
    assert int(got["sizeof_mlp_launch"]) == ctypes.sizeof(q.qpn_mlp_launch)
    assert int(got["offset_mlp_launch_stream_after"]) == q.qpn_mlp_launch.stream_after.offset
    assert int(got["max_m"]) == q.QPN_MAX_M
    w = _w(n=34816, k=5120)
    p = q.qpn_gemm_plan(w, 1)
    assert [int(v) for v in got["plan_gate_up_m1"].split()] == [
        p.split_k, p.waves_per_group, p.depth, p.k_slices, p.epilogue, p.x_stage, p.whole_groups]
    assert int(got["workspace_gate_up_m8"]) == q.qpn_workspace_bytes(w, 8)


def test_status_strings():
    assert q.qpn_status_string(q.QPN_OK) == "ok"
    assert q.qpn_status_string(q.QPN_ERR_BUFFER_TOO_SMALL) == "buffer too small"
    assert q.qpn_status_string(-99) == "unknown status"


def test_packed_bytes():
    assert q.qpn_packed_bytes(q.QPN_FMT_NVFP4, 512, 1024) == 32 * 4 * 2304
    assert q.qpn_packed_bytes(q.QPN_FMT_FP8_E4M3, 512, 1024) == 32 * 4 * 4096
    # ragged shapes round up to whole 16 x 256 tiles
    assert q.qpn_packed_bytes(q.QPN_FMT_NVFP4, 17, 48) == 2 * 1 * 2304
    assert q.qpn_packed_bytes(q.QPN_FMT_NVFP4, 34816, 5120) == 2176 * 20 * 2304
    # the 27B gate_up matrix: codes + scales exactly, no padding
    assert q.qpn_packed_bytes(q.QPN_FMT_NVFP4, 34816, 5120) == 34816 * 5120 // 2 + 34816 * 5120 // 16
    assert q.qpn_packed_bytes(q.QPN_FMT_NVFP4, 0, 1024) == 0
    assert q.qpn_packed_bytes(q.QPN_FMT_NVFP4, 16, 24) == 0       # K % 16
    assert q.qpn_packed_bytes(3, 16, 32) == 0                      # unknown format
    assert q.qpn_packed_bytes(q.QPN_FMT_FP8_E4M3, -1, 32) == 0


def test_tensor_scale_helper():
    assert q.qpn_nvfp4_tensor_scale(2688.0) == 1.0
    assert q.qpn_nvfp4_tensor_scale(0.0) == 1.0


# the workspace's control block: 64 x 16 argmax key slots of 8 bytes
CONTROL = 64 * 16 * 8


def _w(fmt=q.QPN_FMT_NVFP4, n=512, k=1024, packed=FAKE, rs=FAKE):
    return q.make_weight(fmt, n, k, packed, 1.0, rs)


def _gemm(x, w, y, m, ws=None, wsb=0, split=0, waves=0, depth=0, k_slices=0, valu_dot=0, x_stage=0):
    launch = q.make_launch(split, waves, depth, k_slices, x_stage=x_stage, valu_dot=valu_dot)
    return q.lib().qpn_gemm_tuned(x, ctypes.byref(w), y, m, ws, wsb, ctypes.byref(launch), None)


def _ws(w, m, split=0, waves=0, depth=0, k_slices=0, x_stage=0):
    return q.qpn_workspace_bytes_tuned(w, m, q.make_launch(split, waves, depth, k_slices, x_stage=x_stage))


def _plan(w, m, **kw):
    try:
        return q.qpn_gemm_plan(w, m, q.make_launch(**kw))
    except q.QpnError as e:
        return e.status


def test_gemm_rejects_bad_arguments_before_any_device_call():
    err = q.QPN_ERR_INVALID_ARG
    assert _gemm(FAKE, _w(), FAKE, 17) == err                 # m > 16
    assert _gemm(FAKE, _w(), FAKE, -1) == err
    assert _gemm(None, _w(), FAKE, 1) == err                  # null x
    assert _gemm(FAKE + 8, _w(), FAKE, 1) == err              # x not 16-byte aligned
    assert _gemm(FAKE, _w(), None, 1) == err                  # null y
    assert _gemm(FAKE, _w(packed=None), FAKE, 1) == err       # null packed
    assert _gemm(FAKE, _w(packed=FAKE + 4), FAKE, 1) == err   # misaligned packed
    assert _gemm(FAKE, _w(k=1000), FAKE, 1) == err            # k % 16
    assert _gemm(FAKE, _w(fmt=9), FAKE, 1) == err             # format
    assert _gemm(FAKE, _w(fmt=q.QPN_FMT_FP8_E4M3, rs=None), FAKE, 1) == err  # FP8 needs row scales
    assert _gemm(FAKE, _w(), FAKE, 1, waves=5) == err
    assert _gemm(FAKE, _w(), FAKE, 1, depth=5) == err
    assert _gemm(FAKE, _w(), FAKE, 1, k_slices=3) == err
    assert _gemm(FAKE, _w(), FAKE, 1, valu_dot=2) == err
    assert _gemm(FAKE, _w(), FAKE, 1, valu_dot=-1) == err
    assert _gemm(FAKE, _w(), FAKE, 1, x_stage=3) == err
    assert _gemm(FAKE, _w(), FAKE, 1, x_stage=-1) == err
    assert _gemm(FAKE, _w(), FAKE, 1, waves=4, k_slices=8) == q.QPN_ERR_UNSUPPORTED
    w = _w()
    w.reserved = 1
    assert _gemm(FAKE, w, FAKE, 1) == err
    bad_scale = q.make_weight(q.QPN_FMT_NVFP4, 512, 1024, FAKE, float("nan"), None)
    assert _gemm(FAKE, bad_scale, FAKE, 1) == err


def test_gemm_empty_problems_are_noops():
    assert _gemm(None, _w(), None, 0) == q.QPN_OK            # m == 0
    assert _gemm(None, _w(n=0), None, 4) == q.QPN_OK         # n == 0


def test_gemm_workspace_checks():
    w = _w(n=5120, k=17408)
    need = q.qpn_workspace_bytes(w, 8)
    assert need > 0                                           # small N splits K
    assert _gemm(FAKE, w, FAKE, 8, None, 0) == q.QPN_ERR_INVALID_ARG
    assert _gemm(FAKE, w, FAKE, 8, FAKE, need - 16) == q.QPN_ERR_BUFFER_TOO_SMALL
    # one counter per n-tile (padded to 256 bytes), the control block, then fp32
    # partials [split][m][n]
    counters = (5120 // 16) * 4
    assert _ws(w, 8, split=5) == (counters + 255) // 256 * 256 + CONTROL + 5 * 8 * 5120 * 4
    # one K range of 17408 x 8 rows does not fit a full activation stage in
    # LDS; the ring stage takes it (and then no workspace is needed)
    full, ring = q.QPN_X_STAGE_FULL, q.QPN_X_STAGE_RING
    assert _ws(w, 8, split=1, x_stage=full) == 0
    assert _gemm(FAKE, w, FAKE, 8, FAKE, need, split=1, x_stage=full) == q.QPN_ERR_UNSUPPORTED
    assert _plan(w, 8, split_k=1).x_stage == ring
    assert _plan(w, 8, split_k=1, x_stage=full) == q.QPN_ERR_UNSUPPORTED
    assert _ws(_w(n=5120, k=4096), 1, split=1) == 0
    assert _ws(_w(n=5120, k=4096), 1, split=1, k_slices=4) == 0     # K slices need no workspace
    # the 27B qkv at M=1 fills the chip without splitting K
    assert q.qpn_workspace_bytes(_w(n=7168, k=5120), 1) == 0
    assert q.qpn_workspace_bytes(_w(), 17) == 0


def test_plan_resolves_tuned_and_rule_based_launches():
    # the 27B gate_up at M=1 comes from the tuned table: 256 whole groups of 8
    # n-tiles, the last 16 groups split K four ways
    p = q.qpn_gemm_plan(_w(n=34816, k=5120), 1)
    assert (p.split_k, p.waves_per_group, p.k_slices, p.depth, p.whole_groups) == (4, 8, 1, 2, 256)
    assert p.x_stage == q.QPN_X_STAGE_RING
    # down at M=1: one K range, full stage
    p = q.qpn_gemm_plan(_w(n=5120, k=17408), 1)
    assert (p.split_k, p.x_stage, p.whole_groups) == (1, q.QPN_X_STAGE_FULL, 0)
    # any other shape goes through the rule: valid values, explicit fields kept
    p = q.qpn_gemm_plan(_w(n=1000, k=3072), 3, q.make_launch(depth=6))
    assert p.depth == 6 and p.waves_per_group in (4, 8) and p.k_slices in (1, 2, 4, 8)
    assert p.waves_per_group % p.k_slices == 0 and p.split_k >= 1
    full, ring = q.QPN_X_STAGE_FULL, q.QPN_X_STAGE_RING
    for m in range(1, 17):
        p = q.qpn_gemm_plan(_w(n=777, k=17408), m)
        assert p.split_k >= 1 and p.waves_per_group in (4, 8) and p.x_stage in (full, ring)
        # a full stage must fit the K range of m rows in LDS
        if p.x_stage == full:
            assert 2 * m * (-(-68 // p.split_k) * 256 + 8) <= 79 * 1024
        else:
            assert p.depth <= 4 and p.k_slices * m <= 4 * p.waves_per_group
    # small M stages the whole K range, from 5 rows on the ring takes over
    assert _plan(_w(n=1000, k=3072), 1).x_stage == full
    assert _plan(_w(n=1000, k=3072), 4).x_stage == full
    assert _plan(_w(n=1000, k=3072), 5).x_stage == ring
    assert _plan(_w(n=1000, k=3072), 8).x_stage == ring
    # the tuned table picks stages per shape and row count
    assert _plan(_w(n=151936, k=5120), 8).x_stage == ring
    assert _plan(_w(n=5120, k=17408), 4).x_stage == ring
    assert _plan(_w(n=5120, k=17408), 2).x_stage == full
    # an automatic stage falls back to what the other fields allow
    assert _plan(_w(n=1000, k=3072), 8, depth=6).x_stage == full
    assert _plan(_w(n=1000, k=3072), 16, waves_per_group=4, k_slices=4).x_stage == full


TABLED = [(q.QPN_FMT_NVFP4, (34816, 5120)), (q.QPN_FMT_NVFP4, (5120, 17408)), (q.QPN_FMT_NVFP4, (7168, 5120)),
          (q.QPN_FMT_NVFP4, (5120, 5120)), (q.QPN_FMT_NVFP4, (151936, 5120)), (q.QPN_FMT_NVFP4, (1792, 5120)),
          (q.QPN_FMT_NVFP4, (5120, 1280)), (q.QPN_FMT_NVFP4, (8704, 5120)), (q.QPN_FMT_NVFP4, (5120, 4352)),
          (q.QPN_FMT_FP8_E4M3, (7168, 5120)), (q.QPN_FMT_FP8_E4M3, (5120, 5120)),
          (q.QPN_FMT_FP8_E4M3, (5120, 17408))]


@pytest.mark.parametrize("fmt,shape", TABLED)
def test_every_tabled_shape_resolves_to_a_valid_plan(fmt, shape):
    """For the shapes the launch table covers, every M = 1..16 (plain, SwiGLU
    where N allows, argmax) resolves to a launch within the kernel's limits:
    a full stage fits the 79 KiB LDS budget, a ring stays within its limits,
    and the workspace covers the split. An uneven grid (9 wavefronts) takes
    NVFP4, the fp16 or fp32 epilogue, one K slice and no split, and at most 9
    n-tiles a workgroup."""
    n, k = shape
    w = q.make_weight(fmt, n, k, FAKE, 1.0, FAKE)
    ku, nt = -(-k // 256), -(-n // 16)
    epis = [q.QPN_EPILOGUE_NONE, q.QPN_EPILOGUE_F32, q.QPN_EPILOGUE_ARGMAX] + (
        [q.QPN_EPILOGUE_SWIGLU] if n % 32 == 0 else [])
    for m in range(1, 17):
        for epi in epis:
            p = q.qpn_gemm_plan(w, m, q.make_launch(epilogue=epi))
            if p.waves_per_group == 9:
                assert fmt == q.QPN_FMT_NVFP4 and epi in (q.QPN_EPILOGUE_NONE, q.QPN_EPILOGUE_F32)
                assert (p.k_slices, p.split_k) == (1, 1) and p.depth in (2, 3)
                assert 1 <= p.whole_groups <= nt and -(-nt // p.whole_groups) <= 9
                assert p.x_stage == q.QPN_X_STAGE_RING or 2 * m * (ku * 256 + 8) <= 79 * 1024
                assert q.qpn_workspace_bytes_tuned(w, m, p) == 0
                continue
            assert p.waves_per_group in (4, 8) and p.k_slices in (1, 2, 4, 8)
            assert p.waves_per_group % p.k_slices == 0 and p.depth in (2, 3, 4, 6, 8)
            ups = -(-ku // p.split_k)
            assert -(-ku // ups) == p.split_k
            groups = -(-nt // (p.waves_per_group // p.k_slices))
            assert 0 <= p.whole_groups <= groups and (p.split_k > 1 or p.whole_groups == 0)
            if p.x_stage == q.QPN_X_STAGE_FULL:
                span = ku if (p.split_k > 1 and p.whole_groups > 0) else ups
                assert 2 * m * (span * 256 + 8) <= 79 * 1024
            else:
                assert p.x_stage == q.QPN_X_STAGE_RING
                assert p.depth <= 4 and p.k_slices * m <= 4 * p.waves_per_group
            if epi == q.QPN_EPILOGUE_SWIGLU:
                assert (p.waves_per_group // p.k_slices) % 2 == 0
            need = q.qpn_workspace_bytes_tuned(w, m, p)
            if p.split_k > 1:
                assert need >= p.split_k * m * n * 4


def test_uneven_grid_plans():
    """The uneven-group grid: whole_groups workgroups of 9 wavefronts share
    the n-tiles (the first NT mod G one more), one K slice, no split. The
    planner takes it for gate_up from 9 rows on with the fp16 or fp32
    epilogue and the shape fields left automatic; everything else keeps the
    tabled split-K grid; explicit requests outside its limits are refused."""
    w = _w(n=34816, k=5120)
    ring = q.QPN_X_STAGE_RING
    fields = lambda p: (p.waves_per_group, p.k_slices, p.split_k, p.depth, p.x_stage, p.whole_groups)  # noqa: E731
    for m in (9, 12, 16):
        assert fields(_plan(w, m)) == (9, 1, 1, 2, ring, 256)
        assert fields(_plan(w, m, epilogue=q.QPN_EPILOGUE_F32)) == (9, 1, 1, 2, ring, 256)
        assert fields(_plan(w, m, x_stage=ring)) == (9, 1, 1, 2, ring, 256)
        assert _ws(w, m) == 0
        for kw in (dict(epilogue=q.QPN_EPILOGUE_SWIGLU), dict(epilogue=q.QPN_EPILOGUE_ARGMAX), dict(depth=3),
                   dict(waves_per_group=8), dict(k_slices=1), dict(split_k=4)):
            p = _plan(w, m, **kw)
            # (a caller's own split keeps all groups split, as on every shape)
            whole, split = (0, 4) if "split_k" in kw else (256, 5)
            assert p.waves_per_group == 8 and p.split_k == split and p.whole_groups == whole, kw
    for m in (1, 4, 8):
        assert _plan(w, m).waves_per_group == 8
    # an explicit request on a tabled shape takes nothing from the rows of
    # the balanced grid (no K split, one slice, depth 2, the stage by M)
    full = q.QPN_X_STAGE_FULL
    assert fields(_plan(w, 1, waves_per_group=9, whole_groups=256)) == (9, 1, 1, 2, full, 256)
    assert fields(_plan(w, 8, waves_per_group=9, whole_groups=256)) == (9, 1, 1, 2, ring, 256)
    assert fields(_plan(w, 16, waves_per_group=9, whole_groups=512, depth=3)) == (9, 1, 1, 3, ring, 512)
    # explicit: NT = 37 n-tiles over 5 workgroups (8, 8, 7, 7, 7 tiles), ragged K
    small = _w(n=16 * 37 - 5, k=304)
    assert fields(_plan(small, 3, split_k=1, waves_per_group=9, depth=2, k_slices=1, x_stage=full,
                        whole_groups=5)) == (9, 1, 1, 2, full, 5)
    assert fields(_plan(small, 16, waves_per_group=9, depth=3, x_stage=ring, whole_groups=37)) == \
        (9, 1, 1, 3, ring, 37)
    bad = q.QPN_ERR_UNSUPPORTED
    for kw in (dict(k_slices=2), dict(split_k=2), dict(whole_groups=0), dict(whole_groups=4),
               dict(whole_groups=38), dict(depth=4), dict(epilogue=q.QPN_EPILOGUE_ARGMAX),
               dict(epilogue=q.QPN_EPILOGUE_SWIGLU), dict(valu_dot=1), dict(block_columns=1)):
        args = dict(waves_per_group=9, whole_groups=5)
        args.update(kw)
        assert _plan(small, 1, **args) in (bad, q.QPN_ERR_INVALID_ARG), kw
    assert _plan(_w(fmt=q.QPN_FMT_FP8_E4M3, n=16 * 37 - 5, k=304), 1, waves_per_group=9, whole_groups=5) == bad
    assert _plan(small, 1, waves_per_group=7, whole_groups=5) in (bad, q.QPN_ERR_INVALID_ARG)


def test_tabled_whole_groups_follow_the_callers_group_size():
    """A tabled whole-group count is meant for the table's n-tiles per
    workgroup: with another workgroup shape it is scaled to keep the same
    n-tiles whole (gate_up at M = 2: 256 groups of 8 tiles, or 512 of 4)."""
    w = _w(n=34816, k=5120)
    p = _plan(w, 2)
    assert (p.waves_per_group, p.k_slices, p.split_k, p.whole_groups) == (8, 1, 4, 256)
    p4 = _plan(w, 2, waves_per_group=4)
    assert (p4.waves_per_group, p4.k_slices, p4.split_k, p4.whole_groups) == (4, 1, 4, 512)
    p4s = _plan(w, 2, waves_per_group=4, epilogue=q.QPN_EPILOGUE_SWIGLU)
    assert p4s.whole_groups == 512
    # two K slices of 8 wavefronts: groups of 4 tiles again
    assert _plan(w, 2, k_slices=2).whole_groups == 512
    # an explicit count is the caller's and is kept
    assert _plan(w, 2, waves_per_group=4, split_k=4, whole_groups=100).whole_groups == 100
    # the entry already has 8-tile groups: nothing to scale
    assert _plan(w, 1, waves_per_group=8).whole_groups == 256


def test_valu_dot_plans_and_checks():
    """The VALU packed-dot path: m <= 4, plain epilogue, full stage, depth
    2..4; never chosen automatically."""
    unsup = q.QPN_ERR_UNSUPPORTED
    w = _w(n=34816, k=5120)
    for m in range(1, 17):
        assert _plan(w, m).valu_dot == 0
    for m in (1, 2, 3, 4):
        p = _plan(w, m, valu_dot=1)
        assert p.valu_dot == 1 and p.x_stage == q.QPN_X_STAGE_FULL and p.depth <= 4
    assert _plan(w, 5, valu_dot=1) == unsup
    assert _plan(w, 1, valu_dot=1, x_stage=q.QPN_X_STAGE_RING) == unsup
    assert _plan(w, 1, valu_dot=1, depth=6) == unsup
    assert _plan(w, 1, valu_dot=1, epilogue=q.QPN_EPILOGUE_F32) == unsup
    assert _plan(w, 1, valu_dot=1, epilogue=q.QPN_EPILOGUE_SWIGLU) == unsup
    assert _plan(w, 1, valu_dot=1, epilogue=q.QPN_EPILOGUE_ARGMAX) == unsup
    # a long K at m = 4 splits so that the full stage fits
    p = _plan(_w(n=5120, k=17408), 4, valu_dot=1)
    assert p.x_stage == q.QPN_X_STAGE_FULL and 2 * 4 * (-(-68 // p.split_k) * 256 + 8) <= 79 * 1024


def test_block_columns_plans_and_checks():
    """Block columns: one activation row of NVFP4 weights with a full stage,
    only on request (1); 0 and 2 leave it off, other values are refused."""
    unsup, err = q.QPN_ERR_UNSUPPORTED, q.QPN_ERR_INVALID_ARG
    full, ring = q.QPN_X_STAGE_FULL, q.QPN_X_STAGE_RING
    w = _w(n=5120, k=17408)
    assert _plan(w, 1, x_stage=full).block_columns == 2
    assert _plan(w, 1, x_stage=full, block_columns=2).block_columns == 2
    assert _plan(w, 1, x_stage=full, block_columns=1).block_columns == 1
    for m in range(2, 17):
        assert _plan(w, m).block_columns == 2
        assert _plan(w, m, block_columns=1) == unsup
    assert _plan(w, 1, x_stage=ring).block_columns == 2
    assert _plan(w, 1, x_stage=ring, block_columns=1) == unsup
    assert _plan(w, 1, valu_dot=1).block_columns == 2
    assert _plan(w, 1, valu_dot=1, block_columns=1) == unsup
    w8 = _w(fmt=q.QPN_FMT_FP8_E4M3, n=5120, k=17408)
    assert _plan(w8, 1, x_stage=full).block_columns == 2
    assert _plan(w8, 1, x_stage=full, block_columns=1) == unsup
    for e in (q.QPN_EPILOGUE_F32, q.QPN_EPILOGUE_SWIGLU, q.QPN_EPILOGUE_ARGMAX):
        assert _plan(w, 1, x_stage=full, epilogue=e).block_columns == 2
        assert _plan(w, 1, x_stage=full, epilogue=e, block_columns=1).block_columns == 1
    # the zero region the B operand reads is part of the LDS budget: a full
    # stage that fills the budget has no room for it
    assert _plan(_w(n=512, k=157 * 256), 1, x_stage=full, split_k=1).block_columns == 2
    assert _plan(_w(n=512, k=157 * 256), 1, x_stage=full, split_k=1, block_columns=1) == unsup
    for bad in (3, -1):
        assert _plan(w, 1, block_columns=bad) == err
        launch = q.make_launch(block_columns=bad)
        assert q.lib().qpn_gemm_tuned(FAKE, ctypes.byref(w), FAKE, 1, None, 0, ctypes.byref(launch), None) == err


def test_whole_groups_plans():
    unsup, err = q.QPN_ERR_UNSUPPORTED, q.QPN_ERR_INVALID_ARG
    ring, full = q.QPN_X_STAGE_RING, q.QPN_X_STAGE_FULL
    w = _w(n=34816, k=5120)                      # 1088 groups of two tiles at waves 4, k_slices 2
    p = _plan(w, 8, split_k=4, waves_per_group=4, k_slices=2, whole_groups=1024, x_stage=ring)
    assert (p.split_k, p.whole_groups) == (4, 1024)
    # more than there are: every group whole (the split stays, with nothing to split)
    assert _plan(w, 8, split_k=4, waves_per_group=4, k_slices=2, whole_groups=5000, x_stage=ring).whole_groups == 1088
    # without a split every group is whole anyway
    assert _plan(w, 8, split_k=1, waves_per_group=4, k_slices=2, whole_groups=7, x_stage=ring).whole_groups == 0
    # the partials workspace does not depend on it
    assert _ws(w, 8, split=4, waves=4, k_slices=2, x_stage=ring) == \
        q.qpn_workspace_bytes_tuned(w, 8, q.make_launch(4, 4, 0, 2, x_stage=ring, whole_groups=1024))
    # a whole group stages all of K: a full stage of 8 x 5120 does not fit LDS
    assert _plan(w, 8, split_k=4, waves_per_group=4, k_slices=2, whole_groups=16, x_stage=full) == unsup
    assert _plan(w, 8, split_k=4, waves_per_group=4, k_slices=2, x_stage=full).x_stage == full
    assert _plan(w, 1, split_k=4, waves_per_group=4, k_slices=2, whole_groups=16, x_stage=full).whole_groups == 16
    launch = q.make_launch(4, 4, 0, 2, whole_groups=-1)
    assert q.lib().qpn_gemm_tuned(FAKE, ctypes.byref(w), FAKE, 8, FAKE, 1 << 30, ctypes.byref(launch), None) == err


def test_ring_stage_limits():
    unsup = q.QPN_ERR_UNSUPPORTED
    ring = q.QPN_X_STAGE_RING
    w = _w(n=1000, k=3072)
    # depth 2..4 only
    for d in (2, 3, 4):
        assert _plan(w, 8, depth=d, x_stage=ring).depth == d
    for d in (6, 8):
        assert _plan(w, 8, depth=d, x_stage=ring) == unsup
    # at most two x pieces per thread: k_slices * m <= 4 * waves
    assert _plan(w, 16, waves_per_group=4, k_slices=1, x_stage=ring).x_stage == ring
    assert _plan(w, 16, waves_per_group=4, k_slices=2, x_stage=ring) == unsup
    assert _plan(w, 16, waves_per_group=8, k_slices=2, x_stage=ring).x_stage == ring
    assert _plan(w, 16, waves_per_group=8, k_slices=4, x_stage=ring) == unsup
    assert _plan(w, 1, waves_per_group=4, k_slices=4, x_stage=ring).x_stage == ring
    # x offsets are 32-bit: 2 * m * k must stay below 2^31
    big = _w(n=16, k=(1 << 26))
    assert _plan(big, 16, x_stage=ring) == unsup
    # the ring needs no split: any K range at any M
    p = _plan(_w(n=5120, k=17408), 16, split_k=1, waves_per_group=8, k_slices=2, x_stage=ring)
    assert (p.split_k, p.x_stage) == (1, ring)
    assert _ws(_w(n=5120, k=17408), 16, split=1, waves=8, k_slices=2, x_stage=ring) == 0


def test_swiglu_epilogue_plans_and_checks():
    # gate_up at M=1 is tuned for one n-tile per workgroup; SwiGLU pairs gate
    # and up tiles, so the resolved shape has an even number of them
    sw = q.make_launch(epilogue=q.QPN_EPILOGUE_SWIGLU)
    p = q.qpn_gemm_plan(_w(n=34816, k=5120), 1, sw)
    assert p.epilogue == q.QPN_EPILOGUE_SWIGLU
    assert (p.waves_per_group // p.k_slices) % 2 == 0
    for m in (1, 2, 4, 8, 16):
        p = q.qpn_gemm_plan(_w(n=1056, k=2304), m, sw)
        assert (p.waves_per_group // p.k_slices) % 2 == 0
    # up to 8 rows the split (and so the workspace) is the plain GEMM's; from
    # 9 rows on the plain GEMM takes the uneven grid and needs none, while
    # SwiGLU keeps its split tail and its own workspace
    w = _w(n=34816, k=5120)
    assert q.qpn_workspace_bytes_tuned(w, 4, sw) == q.qpn_workspace_bytes(w, 4) > 0
    assert q.qpn_workspace_bytes(w, 9) == 0 and q.qpn_workspace_bytes_tuned(w, 9, sw) > 0
    # N must split into two halves of whole 16-row tiles
    assert q.lib().qpn_gemm_swiglu(FAKE, ctypes.byref(_w(n=48, k=256)), FAKE, 1, None, 0, None) == \
        q.QPN_ERR_INVALID_ARG
    # an explicit shape with an odd number of n-tiles per workgroup is refused
    bad = q.make_launch(1, 4, 3, 4, q.QPN_EPILOGUE_SWIGLU)
    assert q.lib().qpn_gemm_tuned(FAKE, ctypes.byref(_w(n=512, k=1024)), FAKE, 1, None, 0,
                                  ctypes.byref(bad), None) == q.QPN_ERR_UNSUPPORTED
    # unknown epilogue values are argument errors
    odd = q.make_launch(epilogue=2)
    assert q.lib().qpn_gemm_tuned(FAKE, ctypes.byref(_w()), FAKE, 1, None, 0, ctypes.byref(odd), None) == \
        q.QPN_ERR_INVALID_ARG


def test_packed_size_limit():
    """The kernel's unit offsets are 32-bit: a weight whose packed form
    reaches 2 GiB is refused before any device work, one n-tile less is
    planned (the GPU test runs those largest weights)."""
    unsup = q.QPN_ERR_UNSUPPORTED
    for fmt, n_ok in ((q.QPN_FMT_NVFP4, 233008), (q.QPN_FMT_FP8_E4M3, 131056)):
        k = 16384
        assert q.qpn_packed_bytes(fmt, n_ok, k) < 2 ** 31 <= q.qpn_packed_bytes(fmt, n_ok + 16, k)
        for m in (1, 8, 16):
            assert isinstance(_plan(_w(fmt, n_ok, k), m), q.qpn_launch)
            assert _plan(_w(fmt, n_ok + 16, k), m) == unsup
            assert q.qpn_workspace_bytes(_w(fmt, n_ok + 16, k), m) == 0
        big = _w(fmt, n_ok + 16, k)
        assert q.lib().qpn_gemm(FAKE, ctypes.byref(big), FAKE, 1, FAKE, 1 << 30, None) == unsup
        assert q.lib().qpn_gemm_f32(FAKE, ctypes.byref(big), FAKE, 1, FAKE, 1 << 30, None) == unsup


def test_f32_epilogue_plans_and_checks():
    # the fp32 output changes no launch choice: shape and workspace are the
    # plain GEMM's, for tuned and rule-based shapes alike
    f32 = q.make_launch(epilogue=q.QPN_EPILOGUE_F32)
    for (n, k) in ((5120, 17408), (5120, 4352), (34816, 5120), (300, 5120), (37, 48)):
        w = _w(n=n, k=k)
        for m in (1, 2, 5, 8, 16):
            a, b = q.qpn_gemm_plan(w, m), q.qpn_gemm_plan(w, m, f32)
            assert b.epilogue == q.QPN_EPILOGUE_F32
            b.epilogue = a.epilogue
            assert bytes(a) == bytes(b), (n, k, m)
            assert q.qpn_workspace_bytes_tuned(w, m, f32) == q.qpn_workspace_bytes(w, m)
    # fp32 output: 4-byte alignment, checked before any device work
    w = _w(n=48, k=256)
    assert q.lib().qpn_gemm_f32(FAKE, ctypes.byref(w), FAKE + 2, 1, None, 0, None) == q.QPN_ERR_INVALID_ARG
    assert q.lib().qpn_gemm_tuned(FAKE, ctypes.byref(w), FAKE + 2, 1, None, 0, ctypes.byref(f32), None) == \
        q.QPN_ERR_INVALID_ARG
    assert q.lib().qpn_gemm_f32(FAKE, ctypes.byref(w), FAKE, q.QPN_MAX_M + 1, None, 0, None) == \
        q.QPN_ERR_INVALID_ARG
    # a split launch still needs its workspace
    sp = q.make_launch(split_k=2, epilogue=q.QPN_EPILOGUE_F32)
    assert q.lib().qpn_gemm_tuned(FAKE, ctypes.byref(_w(n=512, k=1024)), FAKE, 1, None, 0, ctypes.byref(sp),
                                  None) == q.QPN_ERR_INVALID_ARG
    # epilogue values past the last are argument errors
    bad = q.make_launch(epilogue=q.QPN_EPILOGUE_F32 + 1)
    assert q.lib().qpn_gemm_tuned(FAKE, ctypes.byref(w), FAKE, 1, None, 0, ctypes.byref(bad), None) == \
        q.QPN_ERR_INVALID_ARG
    assert q.qpn_workspace_bytes_tuned(w, 1, bad) == 0


def test_argmax_epilogue_checks_and_workspace():
    am = q.make_launch(epilogue=q.QPN_EPILOGUE_ARGMAX)
    w = _w(n=151936, k=5120)
    p = q.qpn_gemm_plan(w, 1, am)
    assert p.epilogue == q.QPN_EPILOGUE_ARGMAX
    need = q.qpn_workspace_bytes_tuned(w, 1, am)
    # n-tile counters, then the control block of key slots (no split here)
    assert p.split_k == 1
    assert need == (151936 // 16 * 4 + 255) // 256 * 256 + CONTROL
    assert q.qpn_workspace_bytes_tuned(w, 16, am) == need
    idx, val = FAKE, FAKE + 64
    call = q.lib().qpn_gemm_argmax
    assert call(FAKE, ctypes.byref(w), idx, val, 1, None, 0, None, None) == q.QPN_ERR_INVALID_ARG
    assert call(FAKE, ctypes.byref(w), idx, val, 1, FAKE, need - 8, None, None) == q.QPN_ERR_BUFFER_TOO_SMALL
    assert call(FAKE, ctypes.byref(w), idx + 2, val, 1, FAKE, need, None, None) == q.QPN_ERR_INVALID_ARG
    sw = q.make_launch(epilogue=q.QPN_EPILOGUE_SWIGLU)
    assert call(FAKE, ctypes.byref(w), idx, val, 1, FAKE, need, ctypes.byref(sw), None) == q.QPN_ERR_INVALID_ARG
    # the argmax epilogue has two outputs: not through qpn_gemm_tuned
    assert q.lib().qpn_gemm_tuned(FAKE, ctypes.byref(w), FAKE, 1, FAKE, need, ctypes.byref(am), None) == \
        q.QPN_ERR_INVALID_ARG


def test_requantize_rejects_bad_arguments():
    L = q.lib()
    err = q.QPN_ERR_INVALID_ARG
    assert L.qpn_requantize_fp8_nvfp4(FAKE, FAKE, 4, 32, 0.0, FAKE, FAKE, None) == err      # scale 0
    assert L.qpn_requantize_fp8_nvfp4(FAKE, FAKE, 4, 32, float("inf"), FAKE, FAKE, None) == err
    assert L.qpn_requantize_fp8_nvfp4(FAKE, FAKE, 4, 40, 1.0, FAKE, FAKE, None) == err      # k % 16
    assert L.qpn_requantize_fp8_nvfp4(None, FAKE, 4, 32, 1.0, FAKE, FAKE, None) == err
    assert L.qpn_requantize_fp8_nvfp4(FAKE, FAKE, 0, 32, 1.0, None, None, None) == q.QPN_OK  # empty
    assert L.qpn_fp8_absmax(FAKE, FAKE, 4, 32, None, None) == err
    assert L.qpn_fp8_absmax(FAKE, FAKE + 2, 4, 32, FAKE, None) == err                        # misaligned


def test_pack_and_quantize_reject_bad_arguments():
    lib = q.lib()
    nv = q.qpn_packed_bytes(q.QPN_FMT_NVFP4, 32, 64)
    assert lib.qpn_pack_nvfp4(FAKE, FAKE, 32, 64, FAKE, nv - 1, FAKE, None) == q.QPN_ERR_BUFFER_TOO_SMALL
    assert lib.qpn_pack_nvfp4(FAKE, FAKE, 32, 64, FAKE + 8, nv, FAKE, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_pack_nvfp4(None, FAKE, 32, 64, FAKE, nv, FAKE, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_pack_nvfp4(FAKE, FAKE, 32, 40, FAKE, nv, FAKE, None) == q.QPN_ERR_INVALID_ARG
    # the invalid-code counter is required (pack reports invalid codes itself)
    assert lib.qpn_pack_nvfp4(FAKE, FAKE, 32, 64, FAKE, nv, None, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_pack_nvfp4(FAKE, FAKE, 32, 64, FAKE, nv, FAKE + 2, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_pack_nvfp4(None, None, 0, 64, None, 0, None, None) == q.QPN_OK  # empty
    f8 = q.qpn_packed_bytes(q.QPN_FMT_FP8_E4M3, 32, 64)
    assert lib.qpn_pack_fp8(FAKE, 32, 64, FAKE, f8 - 16, FAKE, None) == q.QPN_ERR_BUFFER_TOO_SMALL
    assert lib.qpn_pack_fp8(FAKE, 32, 64, FAKE, f8, None, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_pack_fp8(FAKE, 32, 64, FAKE, f8, FAKE + 1, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_unpack_fp8(FAKE, f8, -2, 64, FAKE, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_quantize_nvfp4(FAKE, 4, 64, 0.0, FAKE, FAKE, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_quantize_nvfp4(FAKE, 4, 64, float("inf"), FAKE, FAKE, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_quantize_fp8(FAKE, 4, 64, FAKE, None, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_absmax_f32(FAKE, -1, FAKE, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_read_ceiling(FAKE, 100, FAKE, 0, 0, None) == q.QPN_ERR_INVALID_ARG  # bytes % 16
    assert lib.qpn_read_ceiling(FAKE, 96, FAKE, 0, 3, None) == q.QPN_ERR_INVALID_ARG   # loads 2, 4 or 8
    assert lib.qpn_read_ceiling(FAKE, 96, FAKE, -1, 4, None) == q.QPN_ERR_INVALID_ARG  # grid


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "quantized_weight_skinny_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


def test_noalloc_checks_before_any_device_call():
    """qpn_gemm_noalloc: argument checks, and a launch needing more than its
    scratch is refused before any HIP call."""
    lib = q.lib()
    w = q.make_weight(q.QPN_FMT_NVFP4, 1024, 1 << 20, FAKE)
    assert q.qpn_workspace_bytes(w, 16) > q.QPN_NOALLOC_SCRATCH_BYTES
    assert lib.qpn_gemm_noalloc(FAKE, ctypes.byref(w), FAKE, 16, None) == q.QPN_ERR_BUFFER_TOO_SMALL
    assert lib.qpn_gemm_noalloc(FAKE, ctypes.byref(w), FAKE, 17, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_gemm_noalloc(FAKE, None, FAKE, 1, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_gemm_noalloc(FAKE, ctypes.byref(_w(fmt=9)), FAKE, 1, None) == q.QPN_ERR_INVALID_ARG
    assert lib.qpn_gemm_noalloc(None, ctypes.byref(_w()), FAKE, 0, None) == q.QPN_OK  # nothing to do


def _mlp_weights(f=17408, k=5120, n=5120, fmt_up=None, fmt_dn=None):
    fu = fmt_up or q.QPN_FMT_NVFP4
    fd = fmt_dn or q.QPN_FMT_NVFP4
    return q.make_weight(fu, 2 * f, k, FAKE, 1.0, FAKE), q.make_weight(fd, n, f, FAKE, 1.0, FAKE)


def _mlp(x, up, dn, h, y, m, ws, ws_bytes, launch=None):
    n = ctypes.c_int32(-1)
    st = q.lib().qpn_mlp(x, ctypes.byref(up), ctypes.byref(dn), h, y, m, ws, ws_bytes,
                         ctypes.byref(launch) if launch is not None else None, ctypes.byref(n), None)
    return st, n.value


def test_mlp_workspace_layout():
    """The two GEMMs' workspaces (each sized for either form) and a 256-byte
    control block at the end; the one-launch form exists for NVFP4 only."""
    up, dn = _mlp_weights()
    for m in (1, 2, 4, 8, 16):
        need = q.qpn_mlp_workspace_bytes(up, dn, m)
        ws_up = max(q.qpn_workspace_bytes_tuned(up, m, q.make_launch(epilogue=q.QPN_EPILOGUE_SWIGLU)),
                    q.qpn_workspace_bytes_tuned(up, m, q.make_launch(epilogue=q.QPN_EPILOGUE_SWIGLU,
                                                                     waves_per_group=8)))
        assert need >= (ws_up + 255) // 256 * 256 + 256
        assert need % 256 == 0
        assert q.qpn_mlp_workspace_bytes(up, dn, m, q.make_mlp_launch(fused=2)) > 0
    f8_up, f8_dn = _mlp_weights(fmt_up=q.QPN_FMT_FP8_E4M3)
    assert q.qpn_mlp_workspace_bytes(f8_up, f8_dn, 1, q.make_mlp_launch(fused=1)) == 0
    assert q.qpn_mlp_workspace_bytes(f8_up, f8_dn, 1) > 0


def test_mlp_argument_checks():
    """Rejected before any device work (no GPU here)."""
    up, dn = _mlp_weights()
    need = q.qpn_mlp_workspace_bytes(up, dn, 1)
    assert _mlp(FAKE, up, dn, FAKE, FAKE, 1, FAKE, need - 16)[0] == q.QPN_ERR_BUFFER_TOO_SMALL
    assert _mlp(FAKE, up, dn, FAKE, FAKE, 1, None, need)[0] == q.QPN_ERR_INVALID_ARG
    assert _mlp(FAKE, up, dn, FAKE + 8, FAKE, 1, FAKE, need)[0] == q.QPN_ERR_INVALID_ARG   # h alignment
    assert _mlp(FAKE + 2, up, dn, FAKE, FAKE, 1, FAKE, need)[0] == q.QPN_ERR_INVALID_ARG   # x alignment
    assert _mlp(FAKE, up, dn, FAKE, FAKE + 1, 1, FAKE, need)[0] == q.QPN_ERR_INVALID_ARG   # y alignment
    assert _mlp(FAKE, up, dn, FAKE, FAKE, 17, FAKE, need)[0] == q.QPN_ERR_INVALID_ARG
    assert _mlp(FAKE, up, dn, FAKE, FAKE, 0, FAKE, need) == (q.QPN_OK, 0)                 # nothing to do
    bad_up, bad_dn = _mlp_weights()
    bad_dn.k = 17392                                                                     # k != n_up / 2
    assert _mlp(FAKE, bad_up, bad_dn, FAKE, FAKE, 1, FAKE, need)[0] == q.QPN_ERR_INVALID_ARG
    for launch in (q.make_mlp_launch(fused=3), q.make_mlp_launch(down_depth=5),
                   q.make_mlp_launch(stream_after=-2), q.qpn_mlp_launch(0, 0, 0, 1)):
        assert _mlp(FAKE, up, dn, FAKE, FAKE, 1, FAKE, need, launch)[0] == q.QPN_ERR_INVALID_ARG
    f8_up, f8_dn = _mlp_weights(fmt_up=q.QPN_FMT_FP8_E4M3)
    need8 = q.qpn_mlp_workspace_bytes(f8_up, f8_dn, 1)
    assert _mlp(FAKE, f8_up, f8_dn, FAKE, FAKE, 1, FAKE, need8, q.make_mlp_launch(fused=1))[0] == \
        q.QPN_ERR_UNSUPPORTED

