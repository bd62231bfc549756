"""Build-level checks on the CPU: the library's sources compile warning-free
with -Wall -Wextra on both the host and the gfx950 pass, the device code holds
no M0 write but the LDS-DMA staging sequence, no packed fp32 arithmetic, no
store through the scalar data cache and no scratch memory or register spills,
and the launch planner and the C ABI's
argument checks run clean under AddressSanitizer and UndefinedBehaviorSanitizer
(a plain host build with g++, driven by tests/host/check_plan.cpp).
"""

import os
import re
import shutil
import subprocess

import pytest

from quantized_weight_skinny_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = qbuild.CSRC
INCLUDE = os.path.join(ROOT, "include")
HIPCC = qbuild.HIPCC
DEVICE_SOURCES = ["qpn_gemm.hip", "qpn_mlp.hip", "qpn_pack.hip", "qpn_api.hip"]
HOST_ONLY_SOURCES = ["qpn_plan.cpp", "qpn_checks.cpp"]

# hipcc flags of the library build minus the output kind
COMMON = [f"--offload-arch={qbuild.ARCH}", "-O3", "-std=c++17", "-Wall", "-Wextra", "-Werror",
          "-Wno-unused-command-line-argument",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE]

needs_hipcc = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    """gfx950 assembly of every device source, compiled in parallel."""
    out = tmp_path_factory.mktemp("asm")
    procs = {}
    for src in DEVICE_SOURCES:
        path = out / (src + ".s")
        cmd = [HIPCC, *COMMON, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(path)]
        procs[src] = (path, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    asm = {}
    for src, (path, proc) in procs.items():
        log, _ = proc.communicate(timeout=600)
        assert proc.returncode == 0, f"{src}: device compile failed or warned:\n{log[-4000:]}"
        assert "warning" not in log, f"{src}: device compile warned:\n{log[-4000:]}"
        asm[src] = path.read_text()
    return asm


def _instructions(text):
    """The instruction lines of an assembly listing (mnemonic and operands)."""
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if not s or s.startswith((".", "//")) or s.endswith(":"):
            continue
        yield s


@needs_hipcc
def test_device_code_m0_only_in_staging(device_asm):
    # M0 is a register the compiler reserves; the staging helper writes it in
    # inline assembly, which is safe only while nothing else uses it. Every
    # write must be the helper's three-instruction sequence.
    total = 0
    for src, text in device_asm.items():
        ins = list(_instructions(text))
        for i, s in enumerate(ins):
            ops = s.split(None, 1)
            if len(ops) < 2:
                continue
            dst = ops[1].split(",")[0].strip()
            if dst != "m0":
                continue
            total += 1
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", s), f"{src}: M0 written by `{s}`"
            assert ins[i + 1] == "s_nop 0", f"{src}: `{s}` not followed by s_nop 0"
            assert ins[i + 2].startswith("global_load_lds_dwordx4 "), f"{src}: `{s}` not followed by the LDS load"
        # and every LDS-DMA load comes right after such a write
        for i, s in enumerate(ins):
            if s.startswith("global_load_lds_"):
                assert re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i - 2]) and ins[i - 1] == "s_nop 0", (
                    f"{src}: `{s}` without its M0 write")
    assert total > 0, "the staging sequence is missing from the device code"


@needs_hipcc
def test_device_code_no_packed_fp32(device_asm):
    pat = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
    for src, text in device_asm.items():
        hits = [s for s in _instructions(text) if pat.search(s)]
        assert not hits, f"{src}: packed fp32 instructions: {hits[:5]}"


@needs_hipcc
def test_device_code_no_scalar_stores(device_asm):
    pat = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")
    for src, text in device_asm.items():
        hits = [s for s in _instructions(text) if pat.search(s)]
        assert not hits, f"{src}: writes through the scalar data cache: {hits[:5]}"


@needs_hipcc
def test_device_code_no_scratch_or_spills(device_asm):
    # every kernel keeps its state in registers and LDS: no private segment
    # (scratch memory per lane) and no register spills
    kernels = 0
    for src, text in device_asm.items():
        for key in (".private_segment_fixed_size", ".sgpr_spill_count", ".vgpr_spill_count"):
            vals = re.findall(re.escape(key) + r":\s+(\d+)", text)
            assert all(v == "0" for v in vals), (src, key, sorted(set(vals)))
        kernels += len(re.findall(r"\.private_segment_fixed_size:", text))
    assert kernels > 100


@needs_hipcc
def test_host_pass_warning_clean():
    for src in DEVICE_SOURCES + HOST_ONLY_SOURCES:
        cmd = [HIPCC, *COMMON, "--cuda-host-only", "-fsyntax-only", os.path.join(CSRC, src)]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        log = res.stdout + res.stderr
        assert res.returncode == 0 and "warning" not in log, f"{src}: host pass warned:\n{log[-4000:]}"


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_planner_and_checks_under_sanitizers(tmp_path):
    exe = tmp_path / "check_plan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", INCLUDE,
           *[os.path.join(CSRC, s) for s in HOST_ONLY_SOURCES],
           os.path.join(ROOT, "tests", "host", "check_plan.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    # verify_asan_link_order=0: the run is fine with another library preloaded
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert out.startswith("ok "), out[-4000:]
    plans = int(out.split()[1])
    assert plans > 1000, out  # the sweep reached the planner's accepting paths
