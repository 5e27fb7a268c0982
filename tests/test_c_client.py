"""libatom used from plain C (tests/c_client/atom_client.c): the program
includes include/atom.h, links libatom.so and the HIP runtime, allocates its
own device buffers and runs a zero-staging ReduceScatter, a staged AllGather
of its outputs and a staged AllReduce. The CPU test compiles it (the header
and the library are consumable from C11 with warnings as errors); the GPU
test runs it on seeded inputs and compares every output with the oracle,
bit for bit."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from reduce_atom_03_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_client", "atom_client.c")
LIBDIR = os.path.join(ROOT, "reduce_atom_03_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(out_dir):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("gcc or the HIP runtime headers are not available")
    if not os.path.exists(os.path.join(LIBDIR, "libatom.so")):
        pytest.skip("libatom.so is not built")
    exe = os.path.join(str(out_dir), "atom_client")
    cmd = [gcc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", LIBDIR, "-latom", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_client_compiles(tmp_path):
    exe = _compile(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("n", [65536, 20003])
def test_c_client_matches_the_oracle(tmp_path, n):
    from tests.gpu_util import require_gpu, say
    require_gpu()
    P = 8
    exe = _compile(tmp_path)
    xs = [synth.mixed_bits(80 + n % 7, r, P * n, synth.BF16, specials=False) for r in range(P)]
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    np.concatenate(xs).astype(np.uint16).tofile(inp)
    say(f"C client: P={P} n={n}")
    r = subprocess.run([exe, str(P), str(n), str(inp), str(outp)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    got = np.fromfile(outp, dtype=np.uint16)
    assert got.size == P * n + 2 * P * P * n
    ys = oracle.reduce_scatter(xs)
    ag = oracle.all_gather(ys)
    ar = oracle.all_reduce(xs)
    want = np.concatenate(list(ys) + list(ag) + list(ar)).astype(np.uint16)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} elements differ, first at {bad[:5]}"
