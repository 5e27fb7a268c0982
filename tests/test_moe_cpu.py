"""The MoE entry points without a GPU: the C structure layout seen by the
binding, scratch sizing, and the host validation that runs before any
launch (invalid shapes, NULL or overlapping buffers, alignment)."""

import ctypes
import os
import subprocess

import pytest

from reduce_atom_03_amd import atom as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = 0x7F0000000000          # fake device addresses: never dereferenced


def fake(n, nbytes, start=BASE, off=0):
    step = ((nbytes + 4095) // 4096 + 1) * 4096
    return [start + i * step + off for i in range(n)]


def test_routing_struct_matches_the_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "atom.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(atom_moe_routing),"
        " offsetof(atom_moe_routing, tokens), offsetof(atom_moe_routing, expert_ids),"
        " offsetof(atom_moe_routing, positions), offsetof(atom_moe_routing, counts),"
        " offsetof(atom_moe_routing, recv_rows), offsetof(atom_moe_routing, scratch));return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    R = A.AtomMoeRouting
    want = [ctypes.sizeof(R), R.tokens.offset, R.expert_ids.offset, R.positions.offset,
            R.counts.offset, R.recv_rows.offset, R.scratch.offset]
    assert got == want


def test_scratch_bytes():
    # P * chunks * E int32, rounded up to 256 bytes; chunks of 256 entries
    assert A.atom_moe_scratch_bytes(8, 256, 8, 512) == 8 * 16 * 256 * 4
    assert A.atom_moe_scratch_bytes(8, 256, 8, 0) == 8 * 1 * 256 * 4
    assert A.atom_moe_scratch_bytes(3, 9, 1, 1) == 256
    assert A.atom_moe_scratch_bytes(4, 4, 1, 1) > 0
    for bad in [(0, 8, 2, 4), (17, 32, 2, 4), (8, 250, 8, 4), (8, 4, 2, 4), (8, 2048, 2, 4),
                (8, 64, 0, 4), (8, 64, 17, 4), (8, 64, 2, -1), (8, 64, 2, (1 << 19) + 1)]:
        assert A.atom_moe_scratch_bytes(*bad) == 0, bad


def routing(P=4, E=8, k=2, T=16, **over):
    n = T * k
    ids = fake(P, 4 * n, BASE)
    pos = fake(P, 4 * n, BASE + (1 << 32))
    rt = A.moe_routing(ids, E, k, pos, BASE + (2 << 32), BASE + (3 << 32), BASE + (4 << 32), T)
    for key, v in over.items():
        setattr(rt, key, v)
    return rt


@pytest.mark.parametrize("field,value", [
    ("nranks", 0), ("nranks", 17), ("num_experts", 6), ("num_experts", 2048), ("num_experts", 2),
    ("topk", 0), ("topk", 17), ("tokens", -1), ("tokens", 1 << 21), ("reserved", 1),
    ("counts", None), ("recv_rows", None), ("scratch", None), ("scratch", BASE + (4 << 32) + 8),
])
def test_route_validation(field, value):
    rt = routing(**{field: value})
    assert A.atom_moe_route(rt, stream=0, check=False) == A.ERR_INVALID_ARG


def test_route_rejects_overlaps_and_null_arrays():
    rt = routing()
    rt.positions = rt.expert_ids                      # positions written over the ids
    assert A.atom_moe_route(rt, stream=0, check=False) == A.ERR_INVALID_ARG
    rt = routing()
    rt.counts = BASE + (1 << 32) + 8                  # counts inside rank 0's positions
    assert A.atom_moe_route(rt, stream=0, check=False) == A.ERR_INVALID_ARG
    rt = routing(expert_ids=None)
    assert A.atom_moe_route(rt, stream=0, check=False) == A.ERR_INVALID_ARG
    assert A.lib.atom_moe_route(None, None) == A.ERR_INVALID_ARG


def _move(combine, rt, src, dst, cap, row, dtype=A.DT_BF16, w=None):
    if combine:
        w = w if w is not None else fake(rt.nranks, 4 * rt.tokens * rt.topk, BASE + (9 << 32))
        return A.atom_moe_combine(rt, src, w, dst, cap, row, dtype, stream=0, check=False)
    return A.atom_moe_dispatch(rt, src, dst, cap, row, dtype, stream=0, check=False)


@pytest.mark.parametrize("combine", [False, True])
def test_move_validation(combine):
    P, T, k, H, cap = 4, 16, 2, 64, 40
    rt = routing(P=P, T=T, k=k)
    rows_src = cap if combine else T
    rows_dst = T if combine else cap
    src = fake(P, 2 * H * rows_src, BASE + (5 << 32))
    dst = fake(P, 2 * H * rows_dst, BASE + (6 << 32))
    assert _move(combine, rt, src, dst, -1, H) == A.ERR_INVALID_ARG
    assert _move(combine, rt, src, dst, cap, 0) == A.ERR_INVALID_ARG
    assert _move(combine, rt, src, dst, cap, H, dtype=7) == A.ERR_INVALID_ARG
    assert _move(combine, rt, src, dst[:1] + [0] * (P - 1), cap, H) == A.ERR_INVALID_ARG
    assert _move(combine, rt, src, [src[0]] + dst[1:], cap, H) == A.ERR_INVALID_ARG    # overlap
    assert _move(combine, rt, src, [dst[0]] * P, cap, H) == A.ERR_INVALID_ARG          # outputs alias
    # 120-byte rows and a buffer 2 bytes off 16-byte alignment pass the host
    # checks (they take the element-wise kernels); with no GPU the launch is
    # what fails. Never launched where a GPU is present: the addresses are fake.
    import torch
    if torch.cuda.device_count() == 0:
        assert _move(combine, rt, src, dst, cap, 60) == A.ERR_HIP
        assert _move(combine, rt, [src[0] + 2] + src[1:], dst, cap, H) == A.ERR_HIP
    assert _move(combine, rt, [src[0] + 1] + src[1:], dst, cap, H) == A.ERR_INVALID_ARG  # not element-aligned
    assert _move(combine, routing(P=P, T=0, k=k), src, dst, cap, H) == A.OK           # nothing to move
    if combine:
        assert _move(True, rt, src, dst, cap, H, w=[BASE + (9 << 32) + 2] * P) == A.ERR_INVALID_ARG
        assert _move(True, rt, src, [rt.positions[0]] + dst[1:], cap, H) == A.ERR_INVALID_ARG


@pytest.mark.parametrize("combine", [False, True])
def test_move_config(combine):
    """cfg: lanes (64-256), stages, num_wgs and ATOM_F_NO_NT apply; the staged
    and XCD-order flags and 512 lanes are unsupported; malformed values are
    invalid. All decided on the host."""
    P, T, k, H, cap = 4, 16, 2, 64, 40
    rt = routing(P=P, T=T, k=k)
    rows_src = cap if combine else T
    rows_dst = T if combine else cap
    src = fake(P, 2 * H * rows_src, BASE + (5 << 32))
    dst = fake(P, 2 * H * rows_dst, BASE + (6 << 32))

    def call(cfg):
        if combine:
            w = fake(P, 4 * T * k, BASE + (9 << 32))
            return A.atom_moe_combine(rt, src, w, dst, cap, H, A.DT_BF16, stream=0, check=False,
                                      cfg=cfg)
        return A.atom_moe_dispatch(rt, src, dst, cap, H, A.DT_BF16, stream=0, check=False, cfg=cfg)

    for flags in (A.F_STAGED, A.F_XCD_ORDER):
        assert call(A.config(flags=flags)) == A.ERR_UNSUPPORTED
    assert call(A.config(lanes=512)) == A.ERR_UNSUPPORTED
    for bad in (A.config(lanes=96), A.config(stages=3), A.config(num_wgs=-1), A.config(flags=0x80)):
        assert call(bad) == A.ERR_INVALID_ARG
