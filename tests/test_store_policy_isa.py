"""Output store policy in the gfx950 assembly (CPU only: hipcc
cross-compiles).

Streaming outputs are written with non-temporal stores unless the caller
passes ATOM_F_NO_NT. Written through a pointer as `nt ? nontemporal store :
store`, the compiler merges the two identical stores into one ordinary store
and drops the hint, so the streaming policy silently disappears (an 8-way
reduce measured 13 % slower on MI355X when the caches held dirty lines).
The kernels therefore store through buffer resources with the policy as an
immediate operand of each branch. This test checks that every zero-staging
and MoE movement vector kernel carries both stores, and that no 16-byte
output store goes through a pointer. (The element-wise fallbacks for
buffers off 16-byte alignment use ordinary stores.)"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduce_atom_03_amd", "csrc")
KERNELS = {"k_reduce.hip": r"k_reduce_vec", "k_copy.hip": r"k_copy_vec",
           "k_moe.hip": r"k_moe_(?:dispatch|combine)I"}   # the vector kernels, not the _elem fallbacks


@pytest.fixture(scope="module", params=sorted(KERNELS))
def asm(request, tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / (request.param + ".s")
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(CSRC, request.param), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-2000:])
    return request.param, out.read_text()


def _kernels(text, pattern):
    out = []
    for m in re.finditer(r"^(_Z\S*%s\S*):" % pattern, text, re.M):
        end = text.find("s_endpgm", m.end())
        out.append((m.group(1), text[m.end():end]))
    return out


def test_output_stores_carry_their_policy(asm):
    src, text = asm
    kernels = _kernels(text, KERNELS[src])
    assert kernels, src
    for name, body in kernels:
        stores = re.findall(r"^\s*(buffer_store_dwordx4[^\n]*)", body, re.M)
        assert any(re.search(r"\bnt\b", op) for op in stores), f"{name}: no non-temporal store"
        assert any(not re.search(r"\b(nt|sc0|sc1)\b", op) for op in stores), \
            f"{name}: no ordinary store (ATOM_F_NO_NT)"
        assert not re.search(r"global_store_dwordx4", body), \
            f"{name}: a 16-byte store through a pointer (policy not an immediate)"
