"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer:
plan.cpp and a randomized driver (tests/plan_fuzz.cpp) built with g++ for
the host only, then run over valid and invalid layouts and configs."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_fuzz"
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    cmd = ["g++", *flags, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "reduce_atom_03_amd", "csrc", "plan.cpp"),
           os.path.join(ROOT, "tests", "plan_fuzz.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), "20000"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "0 failures" in r.stdout
