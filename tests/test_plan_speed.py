"""Host planning stays negligible next to a launch: planning the decode
AllReduce (8 x b x 7168 bf16) and the 8 x 4096-row AllToAllV, in C++ built
with g++ -O2, must take well under a microsecond per call."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planning_takes_well_under_a_microsecond(tmp_path):
    exe = tmp_path / "plan_speed"
    cmd = ["g++", "-std=c++17", "-O2", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "reduce_atom_03_amd", "csrc", "plan.cpp"),
           os.path.join(ROOT, "tests", "plan_speed.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120).stdout
    ns = {line.split()[0]: float(line.split()[1]) for line in out.splitlines() if line.strip()}
    print(ns)
    assert set(ns) == {"allreduce_b1", "allreduce_b16", "alltoallv"}
    assert all(0 < v < 1000 for v in ns.values()), ns
