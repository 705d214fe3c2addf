"""The lattice step's host plan (csrc/plan.h: configuration checks, workspace
carving, rows per round, per-sequence plans, attention items and block lists,
HIP-graph key, FSM update) built alone by the host compiler with
AddressSanitizer and UndefinedBehaviorSanitizer, and run over enumerated and
random states (tests/host/plan_check.cpp states the facts it checks)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs the host C++ compiler")
def test_host_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-DDEX_HD=", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "lossless_depth_adaptive_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "plan_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "plan checks ok" in r.stdout
