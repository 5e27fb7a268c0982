"""The C ABI without a GPU: the library loads and exports every declared
symbol; validation and planning (which run before any HIP call) return the
documented codes and plans; the BDP helper reproduces Table 3."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

from reduce_atom_03_amd import atom as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = 0x7F0000000000          # fake device addresses: never dereferenced
MiB = 1 << 20


def fake(P, nbytes, start=BASE, align_off=0):
    """P disjoint fake device buffers of nbytes each."""
    step = ((nbytes + 4095) // 4096 + 1) * 4096
    return [start + r * step + align_off for r in range(P)]


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "atom.h")).read()
    declared = set(re.findall(r"^\w[\w\s\*]*?\b(atom_\w+)\s*\(", hdr, re.M))
    assert {"atom_copy", "atom_reduce", "atom_collective"} <= declared
    lib = ctypes.CDLL(A.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), f"libatom does not export {name}"
    assert declared == set(A.EXPORTS)


def test_status_strings_and_version():
    for s in range(6):
        assert A.atom_status_string(s) not in ("", "unknown status")
    assert A.atom_status_string(99) == "unknown status"
    assert A.atom_version() >= 1


def test_bdp_reproduces_table3(golden_dir):
    with open(os.path.join(golden_dir, "table3_bdp.json")) as f:
        rows = json.load(f)["rows"]
    for row in rows:
        assert A.atom_bdp_chunk_bytes(row["R_bytes_per_s"], row["tau_s"]) == row["bdp_bytes"], row
        # the printed R*tau column rounds the same way
        assert A.atom_bdp_chunk_bytes(row["rtau_printed_bytes"], 1.0) == row["bdp_bytes"], row


def test_bdp_edges():
    assert A.atom_bdp_chunk_bytes(0, 1e-6) == 0
    assert A.atom_bdp_chunk_bytes(-1, 1) == 0
    assert A.atom_bdp_chunk_bytes(float("nan"), 1) == 0
    assert A.atom_bdp_chunk_bytes(3 * MiB, 1.0) == 4 * MiB      # tie goes up
    assert A.atom_bdp_chunk_bytes(MiB, 1.0) == MiB
    assert A.atom_bdp_chunk_bytes(MiB + 1, 1.0) == MiB


# ---------------------------------------------------------------- validation

def test_copy_validation():
    assert A.atom_copy(0, 0, 0, stream=0, check=False) == A.OK     # nothing to do
    assert A.atom_copy(0, BASE, 16, stream=0, check=False) == A.ERR_INVALID_ARG
    assert A.atom_copy(BASE, 0, 16, stream=0, check=False) == A.ERR_INVALID_ARG
    assert A.atom_copy(BASE + 8, BASE, 16, stream=0, check=False) == A.ERR_INVALID_ARG
    assert A.atom_copy(BASE, BASE + 8, 16, stream=0, check=False) == A.ERR_INVALID_ARG


def test_reduce_validation():
    s = fake(3, 64)
    d = fake(1, 64, start=BASE + (1 << 32))[0]
    R = lambda *a, **k: A.atom_reduce(*a, stream=0, check=False, **k)
    assert R(d, s, 0, dtype=A.DT_BF16) == A.OK                      # zero count
    assert R(d, [], 4, dtype=A.DT_BF16) == A.ERR_INVALID_ARG
    assert R(d, fake(17, 64), 4, dtype=A.DT_BF16) == A.ERR_INVALID_ARG
    assert R(d, s, -1, dtype=A.DT_BF16) == A.ERR_INVALID_ARG
    assert R(d, s, 4, dtype=7) == A.ERR_INVALID_ARG
    assert R(d, s, 4, dtype=A.DT_BF16, op=5) == A.ERR_INVALID_ARG
    assert R(d, s, 4, dtype=A.DT_BF16, op=A.OP_COPY) == A.ERR_UNSUPPORTED
    assert R(d + 1, s, 4, dtype=A.DT_BF16) == A.ERR_INVALID_ARG     # not element-aligned
    assert R(d + 2, s, 4, dtype=A.DT_F32) == A.ERR_INVALID_ARG
    assert R(s[1] + 2, s, 4, dtype=A.DT_BF16) == A.ERR_INVALID_ARG  # dst overlaps a source
    assert R(d, [s[0], 0], 4, dtype=A.DT_BF16) == A.ERR_INVALID_ARG


def Q(kin, kout, op, P=4, n=64, ins=None, outs=None, cfg=None, counts=None, row=1,
      dtype=A.DT_BF16, in_counts=True):
    es = 2 if dtype == A.DT_BF16 else 4
    ins = ins if ins is not None else fake(P, P * n * es * 4)
    outs = outs if outs is not None else fake(P, P * n * es * 4, start=BASE + (1 << 36))
    li = A.layout(kin, ins, n, counts if in_counts else None, row, dtype=dtype)
    lo = A.layout(kout, outs, n, None, row, dtype=dtype)
    return A.atom_plan_query(li, lo, op, cfg)


def test_collective_derivation():
    cases = {
        (A.PARTITIONED, A.SHARD, A.OP_SUM): A.COLL_REDUCE_SCATTER,
        (A.SHARD, A.GATHERED, A.OP_COPY): A.COLL_ALL_GATHER,
        (A.PARTITIONED, A.TRANSPOSED, A.OP_COPY): A.COLL_ALL_TO_ALL,
        (A.PARTITIONED, A.GATHERED, A.OP_SUM): A.COLL_ALL_REDUCE,
    }
    for kin in range(4):
        for kout in range(4):
            for op in (A.OP_COPY, A.OP_SUM):
                st, info = Q(kin, kout, op)
                want = cases.get((kin, kout, op))
                if want is None:
                    assert st == A.ERR_UNSUPPORTED, (kin, kout, op)
                else:
                    assert st == A.OK and info.kind == want, (kin, kout, op, st)


def test_v_derivation():
    P = 4
    C = np.arange(P * P, dtype=np.int64).reshape(P, P)
    st, info = Q(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, P=P, counts=C, row=8)
    assert st == A.OK and info.kind == A.COLL_ALL_TO_ALL_V
    assert info.elems_per_rank_in == int(C[0].sum()) * 8
    for j in range(P):
        assert info.elems_per_rank_out[j] == int(C[:, j].sum()) * 8
    cnt = np.array([3, 0, 5, 1], dtype=np.int64)
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=P, counts=cnt, row=2)
    assert st == A.OK and info.kind == A.COLL_REDUCE_SCATTER_V
    assert [info.elems_per_rank_out[k] for k in range(P)] == [6, 0, 10, 2]
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=P, counts=cnt, row=2)
    assert st == A.OK and info.kind == A.COLL_ALL_GATHER_V
    assert info.elems_per_rank_out[0] == 18
    # AllReduce has no V form
    st, _ = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=P, counts=cnt, row=2)
    assert st == A.ERR_UNSUPPORTED


def test_collective_validation_errors():
    P = 4
    ins = fake(P, 4096)
    outs = fake(P, 4096, start=BASE + (1 << 36))
    ok = lambda st: st[0]
    # mismatched rank counts
    li = A.layout(A.PARTITIONED, ins, 64, dtype=A.DT_BF16)
    lo = A.layout(A.SHARD, outs[:3], 64, dtype=A.DT_BF16)
    assert A.atom_plan_query(li, lo, A.OP_SUM)[0] == A.ERR_INVALID_ARG
    # too many ranks
    li = A.layout(A.PARTITIONED, fake(17, 4096), 64, dtype=A.DT_BF16)
    lo = A.layout(A.SHARD, fake(17, 4096, start=BASE + (1 << 36)), 64, dtype=A.DT_BF16)
    assert A.atom_plan_query(li, lo, A.OP_SUM)[0] == A.ERR_INVALID_ARG
    # dtype mismatch
    li = A.layout(A.PARTITIONED, ins, 64, dtype=A.DT_BF16)
    lo = A.layout(A.SHARD, outs, 64, dtype=A.DT_F32)
    assert A.atom_plan_query(li, lo, A.OP_SUM)[0] == A.ERR_INVALID_ARG
    # part size mismatch, negative size
    assert ok(Q(A.PARTITIONED, A.SHARD, A.OP_SUM, n=-1)) == A.ERR_INVALID_ARG
    li = A.layout(A.PARTITIONED, ins, 64, dtype=A.DT_BF16)
    lo = A.layout(A.SHARD, outs, 65, dtype=A.DT_BF16)
    assert A.atom_plan_query(li, lo, A.OP_SUM)[0] == A.ERR_INVALID_ARG
    # misaligned (odd) bf16 pointer
    bad = list(ins)
    bad[2] += 1
    assert ok(Q(A.PARTITIONED, A.SHARD, A.OP_SUM, ins=bad)) == A.ERR_INVALID_ARG
    # output overlapping an input, outputs overlapping each other
    assert ok(Q(A.PARTITIONED, A.SHARD, A.OP_SUM, outs=[ins[0] + 64] + outs[1:])) == A.ERR_INVALID_ARG
    assert ok(Q(A.PARTITIONED, A.SHARD, A.OP_SUM, outs=[outs[0], outs[0] + 64] + outs[2:])) \
        == A.ERR_INVALID_ARG
    # NULL buffer with data
    assert ok(Q(A.PARTITIONED, A.SHARD, A.OP_SUM, ins=[0] + ins[1:])) == A.ERR_INVALID_ARG
    # negative count, count too large for a segment
    C = np.ones((P, P), dtype=np.int64)
    C[1, 2] = -3
    assert ok(Q(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, counts=C, row=4)) == A.ERR_INVALID_ARG
    C[1, 2] = 1 << 31
    assert ok(Q(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, counts=C, row=4)) == A.ERR_INVALID_ARG
    # bad row width
    C[1, 2] = 1
    assert ok(Q(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, counts=C, row=0)) == A.ERR_INVALID_ARG
    # bad op, bad layout kind
    assert ok(Q(A.PARTITIONED, A.SHARD, 9)) == A.ERR_INVALID_ARG
    assert ok(Q(7, A.SHARD, A.OP_SUM)) == A.ERR_INVALID_ARG


@pytest.mark.parametrize("field,value", [
    ("chunk_bytes", 3 * MiB), ("chunk_bytes", 32 << 10), ("chunk_bytes", 32 * MiB),
    ("stages", 3), ("stages", 16), ("num_wgs", -1), ("flags", 0x80), ("ring_slots", 65),
    ("ring_slots", -2), ("piece_bytes", 3000), ("piece_bytes", 8 << 10), ("wait_us", -1),
    ("lanes", 32), ("lanes", 100), ("lanes", 384), ("lanes", 1024), ("lanes", -64)])
def test_config_validation(field, value):
    cfg = A.config(**{field: value})
    assert Q(A.SHARD, A.GATHERED, A.OP_COPY, cfg=cfg)[0] == A.ERR_INVALID_ARG


def test_every_collective_can_be_staged():
    """The abstract: SNAC is the orchestration of every collective. Each
    layout pair plans a staged launch with the matching stage (copy or
    reduce); partitions off 16-byte alignment are accepted and planned on
    the element-wise path."""
    cfg = A.config(flags=A.F_STAGED)
    C = np.arange(16, dtype=np.int64).reshape(4, 4) % 5
    cases = [
        (A.SHARD, A.GATHERED, A.OP_COPY, {}, A.COLL_ALL_GATHER),
        (A.PARTITIONED, A.GATHERED, A.OP_SUM, {}, A.COLL_ALL_REDUCE),
        (A.PARTITIONED, A.SHARD, A.OP_SUM, {}, A.COLL_REDUCE_SCATTER),
        (A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, {}, A.COLL_ALL_TO_ALL),
        (A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, {"counts": C, "row": 8}, A.COLL_ALL_TO_ALL_V),
        (A.PARTITIONED, A.SHARD, A.OP_SUM, {"counts": np.array([3, 0, 5, 1]), "row": 8},
         A.COLL_REDUCE_SCATTER_V),
        (A.SHARD, A.GATHERED, A.OP_COPY, {"counts": np.array([3, 0, 5, 1]), "row": 8},
         A.COLL_ALL_GATHER_V),
    ]
    for lin, lout, op, kw, kind in cases:
        st, info = Q(lin, lout, op, cfg=cfg, **kw)
        assert st == A.OK and info.staged == 1 and info.kind == kind, (lin, lout, op, kw)
        assert info.vector_path == 1
    # 63-element partitions: the outputs' segments off the sources' 16-byte
    # phase, consumed by the shifted path
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, n=63, cfg=cfg)
    assert st == A.OK and info.staged == 1 and info.vector_path == 1 and info.shifted == 1
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, ins=[b + 2 for b in fake(4, 4096)], cfg=cfg)
    assert st == A.OK and info.staged == 1 and info.vector_path == 1 and info.shifted == 1
    # sources of one partition at different offsets: element by element
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, ins=[b + 2 * (r == 1) for r, b in enumerate(fake(4, 4096))],
                 cfg=cfg)
    assert st == A.OK and info.staged == 1 and info.vector_path == 0


def test_jitter_hook_validation():
    for v in (-1, 10001):
        assert Q(A.SHARD, A.GATHERED, A.OP_COPY,
                 cfg=A.config(flags=A.F_STAGED, jitter_us=v))[0] == A.ERR_INVALID_ARG
    for v in (0, 1, 10000):
        assert Q(A.SHARD, A.GATHERED, A.OP_COPY,
                 cfg=A.config(flags=A.F_STAGED, jitter_us=v, jitter_seed=7))[0] == A.OK


# ------------------------------------------------------------------ planning

def test_credited_bytes_of_the_workloads():
    # ReduceScatter, P=4, 4 x 65536 fp32 per input: (P+1) * P * n * 4
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=4, n=65536, dtype=A.DT_F32)
    assert st == A.OK and info.credited_bytes == 5_242_880
    # 8-way reduce of 8 x 256 MiB bf16 and the fused AllReduce of the same
    n = 1 << 24
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=8, n=n)
    assert info.credited_bytes == 2_415_919_104
    st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=8, n=n)
    assert info.credited_bytes == 4_294_967_296
    # AllToAllV of 8 x 4096 x 7168 bf16: 448 MiB read + 448 MiB written
    C = np.full((8, 8), 512, dtype=np.int64)
    st, info = Q(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, P=8, counts=C, row=7168,
                 ins=fake(8, 56 * MiB), outs=fake(8, 56 * MiB, start=BASE + (1 << 40)))
    assert info.credited_bytes == 939_524_096
    # AllGather at S bytes per partition: 72 S
    S = 8 << 10
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=S // 2)
    assert info.credited_bytes == 72 * S
    # decode AllReduce, b=1: 2 * 8 * 14336
    st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=8, n=896)
    assert info.credited_bytes == 229_376


def test_vector_path_selection():
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, n=64)
    assert info.vector_path == 1 and info.shifted == 0
    # partitions off 16 bytes: the sources of each part agree, the outputs
    # start aligned: the shifted vector path
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, n=63)
    assert info.vector_path == 1 and info.shifted == 1
    ins = [b + 2 for b in fake(4, 4096)]                        # bases off 16 bytes, together
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, ins=ins)
    assert st == A.OK and info.vector_path == 1 and info.shifted == 1
    # sources of one part at different offsets: element-wise
    ins = [b + 2 * (r % 2) for r, b in enumerate(fake(4, 4096))]
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, ins=ins)
    assert st == A.OK and info.vector_path == 0
    # copies: AllToAllV rows of 6 bytes and AllGatherV rows of one element
    C = np.arange(16, dtype=np.int64).reshape(4, 4) % 7
    st, info = Q(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, counts=C, row=3)
    assert st == A.OK and info.vector_path == 1 and info.shifted == 1
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, counts=np.array([5, 0, 9, 3]), row=1)
    assert st == A.OK and info.vector_path == 1 and info.shifted == 1
    # a fan-out whose outputs sit at different offsets: element-wise
    outs = [b + 2 * (r % 2) for r, b in enumerate(fake(4, 4096, start=BASE + (1 << 36)))]
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, n=63, outs=outs)
    assert st == A.OK and info.vector_path == 0


def test_snac_chunking():
    for chunk in (512 << 10, MiB, 2 * MiB):
        for S in (8 << 10, 3 * MiB + (64 << 10), 64 * MiB):
            cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk, ring_slots=4)
            st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=S // 2, cfg=cfg,
                         ins=fake(8, S), outs=fake(8, 8 * S, start=BASE + (1 << 40)))
            assert st == A.OK and info.staged == 1
            # a partition smaller than the chunk is one chunk of whole pieces
            # (8 KiB partition: one 8 KiB piece)
            used = chunk if S >= chunk else 8 << 10
            assert info.chunk_bytes == used and info.ring_slots == 4
            assert info.num_chunks == 8 * -(-S // used)


def test_snac_default_chunk_per_collective():
    """Without chunk_bytes: 512 KiB chunks for AllGather, 2 MiB for AllReduce."""
    S = 64 * MiB
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=S // 2, cfg=A.config(flags=A.F_STAGED),
                 ins=fake(8, S), outs=fake(8, 8 * S, start=BASE + (1 << 40)))
    assert st == A.OK and info.chunk_bytes == 512 << 10 and info.ring_slots == 64
    # a copying stage whose largest segment reaches 256 MiB: 2 MiB chunks
    for Sk, chunk in ((128 * MiB, 512 << 10), (256 * MiB - 2, 512 << 10), (256 * MiB, 2 * MiB)):
        st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=Sk // 2, cfg=A.config(flags=A.F_STAGED),
                     ins=fake(8, Sk), outs=fake(8, 8 * Sk, start=BASE + (1 << 40)))
        assert st == A.OK and info.chunk_bytes == chunk, Sk
    st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=8, n=S // 2 // 8,
                 cfg=A.config(flags=A.F_STAGED), ins=fake(8, S),
                 outs=fake(8, S, start=BASE + (1 << 40)))
    assert st == A.OK and info.chunk_bytes == 2 * MiB and info.ring_slots == 16
    # a 24 KiB partition: one chunk of 8 KiB pieces (3 of them)
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=12 << 10, cfg=A.config(flags=A.F_STAGED),
                 ins=fake(8, 24 << 10), outs=fake(8, 8 * (24 << 10), start=BASE + (1 << 40)))
    assert st == A.OK and info.chunk_bytes == 24 << 10 and info.num_chunks == 8
    # a 64 KiB partition: 8 KiB pieces (the smallest chosen); a caller's piece is kept
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=32 << 10, cfg=A.config(flags=A.F_STAGED),
                 ins=fake(8, 64 << 10), outs=fake(8, 8 * (64 << 10), start=BASE + (1 << 40)))
    assert st == A.OK and info.chunk_bytes == 64 << 10
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=12 << 10,
                 cfg=A.config(flags=A.F_STAGED, piece_bytes=16 << 10),
                 ins=fake(8, 24 << 10), outs=fake(8, 8 * (24 << 10), start=BASE + (1 << 40)))
    assert st == A.OK and info.chunk_bytes == 32 << 10


def test_lanes_sets_the_tile_width():
    """lanes picks the workgroup width of the zero-staging kernels; the tile
    (and so the workgroup count) scales with it."""
    grids = {}
    for lanes in (0, 64, 128, 256):
        st, info = Q(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, P=8, n=1 << 20,
                     cfg=A.config(lanes=lanes), ins=fake(8, 16 * MiB),
                     outs=fake(8, 16 * MiB, start=BASE + (1 << 40)))
        assert st == A.OK
        grids[lanes] = info.num_wgs
    assert grids[64] == 2 * grids[128] == 4 * grids[256]


def test_zero_sized_collective_launches_nothing():
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, n=0)
    assert st == A.OK and info.num_wgs == 0 and info.credited_bytes == 0
    li = A.layout(A.PARTITIONED, fake(4, 64), 0, dtype=A.DT_BF16)
    lo = A.layout(A.SHARD, fake(4, 64, start=BASE + (1 << 36)), 0, dtype=A.DT_BF16)
    assert A.atom_collective(li, lo, A.OP_SUM, stream=0, check=False) == A.OK


def test_snac_default_ring_holds_one_onchip_bdp():
    """Without ring_slots the ring holds 32 MiB (HBM rate x notify round
    trip), in at least 4 and at most 64 slots."""
    for chunk, slots in ((512 << 10, 64), (MiB, 32), (2 * MiB, 16), (16 * MiB, 4), (64 << 10, 64)):
        cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk)
        st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=(64 * MiB) // 2, cfg=cfg,
                     ins=fake(8, 64 * MiB), outs=fake(8, 512 * MiB, start=BASE + (1 << 40)))
        assert st == A.OK and info.ring_slots == slots, (chunk, info.ring_slots)


def test_binding_maps_one_hip_runtime():
    """Importing the binding (even before torch) leaves exactly one HIP
    runtime in the process: libatom binds to the one torch brings."""
    import subprocess
    import sys
    code = ("import reduce_atom_03_amd.atom as A, torch\n"
            "print(len(A._hip_runtimes()))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_snac_piece_spreads_medium_messages():
    """Without piece_bytes the task granule is the largest power of two in
    [8 KiB, 32 KiB] (a copying stage; 64 KiB for a reducing one) with
    P * S / piece >= 512 staging tasks."""
    for S, piece in ((64 << 10, 8 << 10), (512 << 10, 8 << 10), (2 * MiB, 32 << 10),
                     (4 * MiB, 32 << 10), (64 * MiB, 32 << 10)):
        st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=S // 2,
                     cfg=A.config(flags=A.F_STAGED, chunk_bytes=16 * MiB), ins=fake(8, S),
                     outs=fake(8, 8 * S, start=BASE + (1 << 40)))
        assert st == A.OK
        # S < 16 MiB chunk: one chunk of S rounded to whole pieces
        want_chunk = 16 * MiB if S >= 16 * MiB else -(-S // piece) * piece
        assert info.chunk_bytes == want_chunk, (S, info.chunk_bytes)
        tasks = 2 * info.num_chunks * (want_chunk // piece)
        # the tagged hand-off (each chunk staged once, up to 16 MiB staged)
        # runs one workgroup per task; through the counts at most 512
        assert info.snac_tagged == (8 * S <= 16 * MiB), (S, info.snac_tagged)
        want = tasks if info.snac_tagged else min(512, tasks)
        assert info.num_wgs == want, (S, info.num_wgs, tasks)


def test_snac_piece_of_a_reducing_stage():
    """A reducing stage's granule goes up to 64 KiB."""
    P = 8
    for S, piece in ((512 << 10, 8 << 10), (8 * MiB, 16 << 10), (64 * MiB, 64 << 10), (256 * MiB, 64 << 10)):
        n = S // 2 // P
        st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=P, n=n,
                     cfg=A.config(flags=A.F_STAGED, chunk_bytes=16 * MiB), ins=fake(P, S),
                     outs=fake(P, S, start=BASE + (1 << 40)))
        assert st == A.OK and info.staged == 1
        per_rank = n * 2
        want_chunk = 16 * MiB if per_rank >= 16 * MiB else -(-per_rank // piece) * piece
        assert info.chunk_bytes == want_chunk, (S, info.chunk_bytes)
        assert info.snac_tasks == 2 * info.num_chunks * (want_chunk // piece), (S, info.snac_tasks)


def test_snac_grid_follows_the_ring_window():
    """Without num_wgs the staged launch uses one workgroup per piece the ring
    can hold (slots * chunk / piece), at most 512; num_wgs overrides it."""
    S = 64 * MiB
    # (default pieces of a copying stage: 32 KiB)
    for chunk, slots, piece, want in ((512 << 10, 0, 0, 512), (64 << 10, 0, 0, 128),
                                      (256 << 10, 0, 0, 512), (512 << 10, 8, 0, 128),
                                      (2 * MiB, 8, 32 << 10, 512), (1 * MiB, 4, 16 << 10, 256)):
        cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk, ring_slots=slots, piece_bytes=piece)
        st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=S // 2, cfg=cfg, ins=fake(8, S),
                     outs=fake(8, 8 * S, start=BASE + (1 << 40)))
        assert st == A.OK and info.num_wgs == want, (chunk, slots, piece, info.num_wgs)
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, num_wgs=300)
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, n=S // 2, cfg=cfg, ins=fake(8, S),
                 outs=fake(8, 8 * S, start=BASE + (1 << 40)))
    assert st == A.OK and info.num_wgs == 300


def test_wide_workgroups_only_for_the_staged_kernel():
    """512 lanes exist only for the staged kernel: accepted with
    ATOM_F_STAGED, ATOM_ERR_UNSUPPORTED for the zero-staging kernels."""
    for lanes in (512,):
        assert Q(A.SHARD, A.GATHERED, A.OP_COPY, cfg=A.config(lanes=lanes))[0] == A.ERR_UNSUPPORTED
        assert Q(A.PARTITIONED, A.SHARD, A.OP_SUM, cfg=A.config(lanes=lanes))[0] == A.ERR_UNSUPPORTED
        for op, lin in ((A.OP_COPY, A.SHARD), (A.OP_SUM, A.PARTITIONED)):
            st, info = Q(lin, A.GATHERED, op, cfg=A.config(flags=A.F_STAGED, lanes=lanes))
            assert st == A.OK and info.staged == 1, (lanes, op)


def test_coaligned_offsets_plan_the_vector_path():
    """Buffers all off 16-byte alignment by the same amount (and partitions
    of 16-byte multiples) take the vector path with element-wise heads;
    outputs off by a different amount, or partitions that change the offset,
    take the shifted vector path."""
    P, n = 8, 4096
    big = P * n * 2 * 4
    for off in (2, 6, 14):
        ins = fake(P, big, align_off=off)
        outs = fake(P, big, start=BASE + (1 << 36), align_off=off)
        for kin, kout, op in ((A.PARTITIONED, A.SHARD, A.OP_SUM), (A.PARTITIONED, A.GATHERED, A.OP_SUM),
                              (A.SHARD, A.GATHERED, A.OP_COPY), (A.PARTITIONED, A.TRANSPOSED, A.OP_COPY)):
            st, info = Q(kin, kout, op, P=P, n=n, ins=ins, outs=outs)
            assert st == A.OK and info.vector_path == 1, (off, kin, kout)
        st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=P, n=n, ins=ins,
                     outs=fake(P, big, start=BASE + (1 << 36), align_off=(off + 2) % 16))
        assert st == A.OK and info.vector_path == 1 and info.shifted == 1
        st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=P, n=n + 1, ins=ins, outs=outs)
        assert st == A.OK and info.vector_path == 1 and info.shifted == 1  # partition k moves the offset


def _plan(kin, kout, op, P, n, in_bytes, out_bytes, cfg=None):
    st, info = Q(kin, kout, op, P=P, n=n, cfg=cfg, ins=fake(P, in_bytes),
                 outs=fake(P, out_bytes, start=BASE + (1 << 40)))
    assert st == A.OK
    return info


def test_launch_shapes_and_store_policy():
    """The planner's measured defaults on MI355X: 64-lane one-tile workgroups
    for the 8-way reduce (1 slot per lane), the fused AllReduce (1) and
    AllToAll (2); 128 lanes x 2 slots for a flat copy; 512 lanes for staged
    calls. Outputs of large messages are written with streaming stores,
    those of the latency path (< 1 MiB per stream) with ordinary ones, and
    ATOM_F_NO_NT makes every store ordinary."""
    P, big = 8, 256 * MiB
    rs = _plan(A.PARTITIONED, A.SHARD, A.OP_SUM, P, big // 2 // P, big, big // P)
    assert (rs.lanes, rs.stages, rs.streaming_stores, rs.grid_rows) == (64, 1, 1, 1)
    assert rs.num_wgs == big // 1024
    ar = _plan(A.PARTITIONED, A.GATHERED, A.OP_SUM, P, big // 2 // P, big, big)
    assert (ar.lanes, ar.stages, ar.streaming_stores) == (64, 1, 1)
    a2a = _plan(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, P, big // 2 // P, big, big)
    assert (a2a.lanes, a2a.stages, a2a.streaming_stores) == (64, 2, 1)
    flat = _plan(A.SHARD, A.GATHERED, A.OP_COPY, 1, big // 2, big, big)
    assert (flat.lanes, flat.stages, flat.streaming_stores) == (128, 2, 1)
    assert flat.num_wgs == big // (128 * 2 * 16)
    ag = _plan(A.SHARD, A.GATHERED, A.OP_COPY, P, 64 * MiB // 2, 64 * MiB, 512 * MiB,
               cfg=A.config(flags=A.F_STAGED))
    assert (ag.staged, ag.lanes, ag.stages, ag.streaming_stores) == (1, 512, 8, 1)
    # zero-staging fan-out beyond the latency path: blocked order, 8 KiB
    # tiles, one workgroup per (tile, output) pair (8 MiB blocks of 1024
    # tiles divide the 8 x 64 MiB exactly)
    agz = _plan(A.SHARD, A.GATHERED, A.OP_COPY, P, 64 * MiB // 2, 64 * MiB, 512 * MiB)
    assert (agz.staged, agz.lanes, agz.stages, agz.streaming_stores) == (0, 256, 2, 1)
    assert agz.num_wgs == P * (P * 64 * MiB // 8192)
    no_nt = _plan(A.PARTITIONED, A.SHARD, A.OP_SUM, P, big // 2 // P, big, big // P,
                  cfg=A.config(flags=A.F_NO_NT))
    assert no_nt.streaming_stores == 0
    # latency path: the decode AllReduce (8 x 7168 bf16) and a small 8-way
    # ReduceScatter; the latter as a tiles x parts grid
    dec = _plan(A.PARTITIONED, A.GATHERED, A.OP_SUM, P, 7168 // P, 7168 * 2, 7168 * 2)
    assert (dec.lanes, dec.stages, dec.streaming_stores, dec.num_wgs) == (64, 1, 0, 14)
    small = _plan(A.PARTITIONED, A.SHARD, A.OP_SUM, P, 4096, P * 8192, 8192)
    assert (small.grid_rows, small.streaming_stores) == (P, 0)
    assert small.num_wgs == P * 8
    ag8 = _plan(A.SHARD, A.GATHERED, A.OP_COPY, P, 4096, 8192, P * 8192)
    assert (ag8.lanes, ag8.stages, ag8.streaming_stores, ag8.num_wgs) == (64, 1, 0, 64)
    assert ag8.grid_rows == P                  # tiles x segments grid
    a2a = _plan(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, P, 512, P * 1024, P * 1024)
    assert (a2a.grid_rows, a2a.num_wgs) == (P * P, P * P)


def test_uniform_grid_only_for_equal_aligned_small_parts():
    """A ReduceScatterV (unequal parts) and any large reduce keep the
    one-dimensional grid that finds each tile's part in the part table."""
    P = 8
    counts = np.array([100, 3, 50, 7, 64, 1, 9, 22], dtype=np.int64)
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=P, n=0, counts=counts, row=8,
                 ins=fake(P, int(counts.sum()) * 16), outs=fake(P, 4096, start=BASE + (1 << 40)))
    assert st == A.OK and info.grid_rows == 1
    big = _plan(A.PARTITIONED, A.SHARD, A.OP_SUM, P, 1 << 21, P * (1 << 22), 1 << 22)
    assert big.grid_rows == 1
    # the same for the copy family: an AllGatherV and a large AllGather
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=P, n=0, counts=counts, row=8,
                 ins=fake(P, 4096), outs=fake(P, int(counts.sum()) * 16, start=BASE + (1 << 40)))
    assert st == A.OK and info.grid_rows == 1
    ag = _plan(A.SHARD, A.GATHERED, A.OP_COPY, P, 1 << 21, 1 << 22, P * (1 << 22))
    assert ag.grid_rows == 1


def _c_layout(tmp_path, struct, fields):
    """sizeof and field offsets of `struct` as the C compiler lays it out."""
    import subprocess
    src = tmp_path / f"{struct}.c"
    fmt = " ".join(["%zu"] * (len(fields) + 1))
    args = ", ".join([f"sizeof({struct})"] + [f"offsetof({struct}, {f})" for f in fields])
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "atom.h"\n'
                   f'int main(void){{printf("{fmt}\\n", {args});return 0;}}\n')
    exe = tmp_path / struct
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    subprocess.run(["gcc", "-I", os.path.join(root, "include"), str(src), "-o", str(exe)], check=True)
    return [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]


@pytest.mark.parametrize("struct,cls", [("atom_config", "AtomConfig"),
                                        ("atom_plan_info", "AtomPlanInfo")])
def test_structs_match_the_header(tmp_path, struct, cls):
    C = getattr(A, cls)
    names = [f[0] for f in C._fields_]
    got = _c_layout(tmp_path, struct, names)
    assert got == [ctypes.sizeof(C)] + [getattr(C, n).offset for n in names]


def test_snac_lead_and_task_count():
    """The ticket order's lead defaults to the ring depth, is clamped to it,
    and out-of-range values are rejected; the task count is 2 * chunks *
    pieces per chunk (the size of the trace array, in quadruples)."""
    ins, outs = fake(8, 8 << 20), fake(8, 64 << 20, start=BASE + (1 << 36))
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=512 << 10, piece_bytes=64 << 10, ring_slots=16)
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, ins=ins, outs=outs, n=(8 << 20) // 2, cfg=cfg)
    assert st == A.OK and info.staged == 1
    assert info.snac_lead == 8
    assert info.snac_tasks == 2 * info.num_chunks * 8
    cfg.snac_lead = 4
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, ins=ins, outs=outs, n=(8 << 20) // 2, cfg=cfg)
    assert st == A.OK and info.snac_lead == 4
    cfg.snac_lead = 40
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, ins=ins, outs=outs, n=(8 << 20) // 2, cfg=cfg)
    assert st == A.OK and info.snac_lead == 16
    for bad in (-1, 65):
        cfg.snac_lead = bad
        st, _ = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, ins=ins, outs=outs, n=(8 << 20) // 2, cfg=cfg)
        assert st == A.ERR_INVALID_ARG, bad
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=8, ins=ins, outs=outs, n=(8 << 20) // 2)
    assert st == A.OK and info.staged == 0 and info.snac_tasks == 0 and info.snac_lead == 0


def test_snac_default_lead_by_stage():
    """Every stage leads by half the ring depth (at least one chunk)."""
    P, n = 8, 1 << 20
    ins = fake(P, P * n * 2)
    outs = fake(P, P * n * 2, start=BASE + (1 << 36))
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=2 << 20, ring_slots=16)
    st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=P, n=n, ins=ins, outs=outs, cfg=cfg)
    assert st == A.OK and info.staged == 1 and info.ring_slots == 16 and info.snac_lead == 8
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=P, n=n, ins=ins, outs=outs, cfg=cfg)
    assert st == A.OK and info.snac_lead == 8
    st, info = Q(A.PARTITIONED, A.TRANSPOSED, A.OP_COPY, P=P, n=n, ins=ins, outs=outs, cfg=cfg)
    assert st == A.OK and info.snac_lead == 8
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=2 << 20, ring_slots=1)
    st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=P, n=n, ins=ins, outs=outs, cfg=cfg)
    assert st == A.OK and info.snac_lead == 1


def test_staged_segments_at_a_common_offset_stay_vectorized():
    """Staged calls: a segment whose streams all sit at one offset from
    16-byte alignment takes the vector path (element-wise ends); one whose
    sources agree and a destination does not is staged the same way and
    consumed by the shifted path; sources at different offsets make the call
    element-wise."""
    P, n = 8, 4096
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=P, n=n, cfg=A.config(flags=A.F_STAGED),
                 ins=fake(P, n * 2, align_off=2), outs=fake(P, P * n * 2, start=BASE + (1 << 36), align_off=2))
    assert st == A.OK and info.staged == 1 and info.vector_path == 1 and info.shifted == 0
    st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=P, n=n, cfg=A.config(flags=A.F_STAGED),
                 ins=fake(P, P * n * 2, align_off=6), outs=fake(P, P * n * 2, start=BASE + (1 << 36), align_off=6))
    assert st == A.OK and info.staged == 1 and info.vector_path == 1 and info.shifted == 0
    # one source per AllGather segment, outputs at another offset: shifted
    st, info = Q(A.SHARD, A.GATHERED, A.OP_COPY, P=P, n=n, cfg=A.config(flags=A.F_STAGED),
                 ins=fake(P, n * 2, align_off=2), outs=fake(P, P * n * 2, start=BASE + (1 << 36), align_off=4))
    assert st == A.OK and info.staged == 1 and info.vector_path == 1 and info.shifted == 1
    # ReduceScatter: the P sources agree, the outputs do not: shifted
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=P, n=n, cfg=A.config(flags=A.F_STAGED),
                 ins=fake(P, P * n * 2, align_off=2), outs=fake(P, n * 2, start=BASE + (1 << 36)))
    assert st == A.OK and info.staged == 1 and info.vector_path == 1 and info.shifted == 1
    # sources at different offsets: element-wise
    ins = fake(P, P * n * 2)
    ins[3] += 2
    st, info = Q(A.PARTITIONED, A.SHARD, A.OP_SUM, P=P, n=n, cfg=A.config(flags=A.F_STAGED),
                 ins=ins, outs=fake(P, n * 2, start=BASE + (1 << 36)))
    assert st == A.OK and info.staged == 1 and info.vector_path == 0


def test_small_aligned_staged_calls_hand_off_through_tagged_words():
    """A staged call whose ring holds every chunk and whose segments each
    have every stream at one offset from 16-byte alignment hands off through
    tagged words, one workgroup per task; ATOM_F_COUNTED, a segment whose
    streams sit at different offsets, a ring too short to hold every
    chunk, a caller's grid or more than 16 MiB staged keep the slot
    counts."""
    P = 8

    def ag(n, cfg, off_in=0, off_out=0):
        return Q(A.SHARD, A.GATHERED, A.OP_COPY, P=P, n=n, cfg=cfg,
                 ins=fake(P, n * 2, align_off=off_in),
                 outs=fake(P, P * n * 2, start=BASE + (1 << 36), align_off=off_out))

    for n in (4096, 65536):          # 8 KiB and 128 KiB per rank
        st, info = ag(n, A.config(flags=A.F_STAGED))
        assert st == A.OK and info.staged == 1 and info.snac_tagged == 1, n
        assert info.num_wgs == info.snac_tasks <= 256
        st, info = ag(n, A.config(flags=A.F_STAGED | A.F_COUNTED))
        assert st == A.OK and info.staged == 1 and info.snac_tagged == 0
        assert info.num_wgs == info.snac_tasks                 # still one workgroup per task
    for reduce_coll in ((A.PARTITIONED, A.GATHERED), (A.PARTITIONED, A.SHARD)):
        st, info = Q(*reduce_coll, A.OP_SUM, P=P, n=512, cfg=A.config(flags=A.F_STAGED))
        assert st == A.OK and info.snac_tagged == 1, reduce_coll
    st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=P, n=512, dtype=A.DT_F32,
                 cfg=A.config(flags=A.F_STAGED))
    assert st == A.OK and info.snac_tagged == 1
    # every stream at one common offset: still tagged (the aligned vectors
    # enclosing each piece are staged); sources and outputs at different
    # offsets (the shifted path): the slot counts
    assert ag(4096, A.config(flags=A.F_STAGED), 2, 2)[1].snac_tagged == 1
    assert ag(4096, A.config(flags=A.F_STAGED), 0, 2)[1].snac_tagged == 0
    # the ticket: a 2-slot ring, or a caller's grid
    st, info = ag(4096, A.config(flags=A.F_STAGED, ring_slots=2))
    assert st == A.OK and info.num_wgs < info.snac_tasks and info.snac_tagged == 0
    st, info = ag(4096, A.config(flags=A.F_STAGED, num_wgs=16))
    assert st == A.OK and info.snac_tagged == 0
    # beyond 256 tasks (256 KiB, 1 MiB and 2 MiB per rank): still one
    # workgroup per task on the tagged ring, which holds 16 MiB of staged data
    for n in (131072, 524288, 1 << 20):
        st, info = ag(n, A.config(flags=A.F_STAGED))
        assert st == A.OK and info.snac_tasks > 256 and info.snac_tagged == 1, n
        assert info.num_wgs == info.snac_tasks
    # through the counts they take the ticket (more than 256 tasks)
    st, info = ag(131072, A.config(flags=A.F_STAGED | A.F_COUNTED))
    assert st == A.OK and info.snac_tasks > 256 and info.snac_tagged == 0
    # more than the tagged ring holds (8 x 4 MiB = 32 MiB staged): the ticket
    st, info = ag(2 << 20, A.config(flags=A.F_STAGED))
    assert st == A.OK and info.snac_tagged == 0 and info.num_wgs < info.snac_tasks
    # a staged AllReduce of 8 MiB per rank stages 8 MiB: tagged
    st, info = Q(A.PARTITIONED, A.GATHERED, A.OP_SUM, P=P, n=(8 << 20) // 2 // P,
                 cfg=A.config(flags=A.F_STAGED))
    assert st == A.OK and info.snac_tagged == 1
    # zero staging ignores the flag
    st, info = ag(4096, A.config(flags=A.F_COUNTED))
    assert st == A.OK and info.staged == 0 and info.snac_tagged == 0
