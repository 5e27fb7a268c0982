"""GPU parity: libatom (through its C ABI) against the CPU oracle, element by
element on the same seeded inputs.

Bars: copies and AllToAll(V) bit-exact; reductions within 1 bf16 ulp
(fp32: relative 1e-6). Both sides accumulate in binary32 in rank order and
round once with round-to-nearest-even, so the reductions are also checked
for bitwise equality where the inputs are finite."""

import numpy as np
import pytest

import oracle
from reduce_atom_03_amd import synth
from tests._helpers import assert_bf16_close, assert_bits_equal, assert_f32_close
from tests.gpu_util import (check_guards, empty_dev, from_dev, out_buffers, require_gpu, say,
                            to_dev)

pytestmark = pytest.mark.gpu

GUARD = 40   # canary elements around every output


@pytest.fixture(scope="module")
def A():
    require_gpu()
    from reduce_atom_03_amd import atom
    return atom


def _torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == synth.BF16 else torch.float32


def _assert_reduced(got, want, what):
    if want.dtype == np.uint16:
        assert_bf16_close(got, want, 1, what)
    else:
        assert_f32_close(got, want, 1e-6, what)
    assert_bits_equal(got, want, what + " (bitwise)")


def _sync():
    import torch
    torch.cuda.synchronize()


# ------------------------------------------------------------- ReduceScatter

@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 4099, 70000])
def test_reduce_scatter(A, P, n, dtype):
    say(f"RS P={P} n={n} {dtype}")
    xs = [synth.mixed_bits(31, r, P * n, dtype, specials=False) for r in range(P)]
    want = oracle.reduce_scatter(xs)
    dx = [to_dev(x)[1] for x in xs]
    fulls, ys = out_buffers([n] * P, _torch_dtype(dtype), GUARD)
    A.reduce_scatter(dx, ys)
    _sync()
    for k in range(P):
        _assert_reduced(from_dev(ys[k]), want[k], f"RS y_{k}")
    check_guards(fulls, [n] * P, GUARD)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
def test_reduce_scatter_specials(A, dtype):
    """Infinities, NaNs, signed zeros and subnormals: NaN results compared by
    class, everything else bitwise."""
    P, n = 8, 3000
    xs = [synth.mixed_bits(32, r, P * n, dtype, specials=True) for r in range(P)]
    want = oracle.reduce_scatter(xs)
    dx = [to_dev(x)[1] for x in xs]
    ys = [empty_dev(n, _torch_dtype(dtype)) for _ in range(P)]
    A.reduce_scatter(dx, ys)
    _sync()
    for k in range(P):
        assert_bits_equal(from_dev(ys[k]), want[k], f"RS specials y_{k}")


def test_reduce_scatter_c1(A):
    """ReduceScatter, P=4, each input 4 x 65536 fp32 U[-1,1] (seed 1)."""
    say("RS c1 P=4 n=65536 f32")
    xs = synth.c1_inputs()
    want = oracle.reduce_scatter(xs)
    dx = [to_dev(x)[1] for x in xs]
    ys = [empty_dev(65536, _torch_dtype(synth.F32)) for _ in range(4)]
    A.reduce_scatter(dx, ys)
    _sync()
    for k in range(4):
        _assert_reduced(from_dev(ys[k]), want[k], f"c1 y_{k}")


def test_reduce_scatter_unaligned(A):
    """Buffers 2 bytes off 16-byte alignment take the element-wise path."""
    P, n = 5, 1031
    xs = [synth.mixed_bits(33, r, P * n, synth.BF16, specials=False) for r in range(P)]
    want = oracle.reduce_scatter(xs)
    dx = [to_dev(x, pad_before=1)[1] for x in xs]
    fulls, ys = out_buffers([n] * P, _torch_dtype(synth.BF16), GUARD + 1)
    ys = [f[GUARD + 1 + 1:GUARD + 2 + n] for f in fulls]          # odd element offset
    A.reduce_scatter(dx, ys)
    _sync()
    for k in range(P):
        _assert_reduced(from_dev(ys[k]), want[k], f"RS unaligned y_{k}")


# ---------------------------------------------------------------- AllReduce

@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("P", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("n", [0, 1, 9, 896, 4099, 33000])
def test_all_reduce(A, P, n, dtype):
    say(f"AR P={P} n={n} {dtype}")
    xs = [synth.mixed_bits(34, r, P * n, dtype, specials=False) for r in range(P)]
    want = oracle.all_reduce(xs)
    dx = [to_dev(x)[1] for x in xs]
    fulls, outs = out_buffers([P * n] * P, _torch_dtype(dtype), GUARD)
    A.all_reduce(dx, outs)
    _sync()
    got0 = from_dev(outs[0])
    _assert_reduced(got0, want[0], "AR out_0")
    for j in range(1, P):
        assert_bits_equal(from_dev(outs[j]), got0, f"AR out_{j} == out_0", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD)


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16])
def test_decode_all_reduce(A, b):
    """Decode AllReduce: 8 buffers of b x 7168 bf16, N(0, 0.02) (seed 5)."""
    say(f"decode AR b={b}")
    xs = synth.c5_inputs(b)
    want = oracle.all_reduce(xs)
    dx = [to_dev(x)[1] for x in xs]
    outs = [empty_dev(b * synth.HIDDEN, _torch_dtype(synth.BF16)) for _ in range(8)]
    A.all_reduce(dx, outs)
    _sync()
    for j in range(8):
        _assert_reduced(from_dev(outs[j]), want[j], f"decode AR b={b} out_{j}")


# ------------------------------------------------------------------ reduce

@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("m", [1, 5, 8, 263, 65541])
def test_reduce(A, P, m, dtype):
    say(f"reduce P={P} m={m} {dtype}")
    xs = [synth.mixed_bits(35, r, m, dtype, specials=False) for r in range(P)]
    want = oracle.reduce(xs)
    dx = [to_dev(x)[1] for x in xs]
    fulls, outs = out_buffers([m], _torch_dtype(dtype), GUARD)
    A.atom_reduce(outs[0], dx)
    _sync()
    _assert_reduced(from_dev(outs[0]), want, "reduce")
    check_guards(fulls, [m], GUARD)


def test_rank_order_on_gpu(A):
    """The rank-order pin, on the device: bf16 (1, 2^-8, 2^-24, 2^-24) must
    give exactly 1.0, fp32 (1, 2^-24, 2^-24, 2^-24) exactly 1.0."""
    import torch
    vals = [1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24]
    xs = [torch.full((64,), v, dtype=torch.bfloat16, device="cuda") for v in vals]
    out = torch.empty(64, dtype=torch.bfloat16, device="cuda")
    A.atom_reduce(out, xs)
    _sync()
    assert (out.float().cpu() == 1.0).all()
    vals = [1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24]
    xs = [torch.full((64,), v, dtype=torch.float32, device="cuda") for v in vals]
    out = torch.empty(64, dtype=torch.float32, device="cuda")
    A.atom_reduce(out, xs)
    _sync()
    assert (out.cpu() == 1.0).all()


# -------------------------------------------------------------------- copy

@pytest.mark.parametrize("nbytes", [0, 2, 16, 30, 4096, 1000002, 4 << 20])
@pytest.mark.parametrize("off", [0, 2])
def test_copy(A, nbytes, off):
    say(f"copy {nbytes} B off={off}")
    n = nbytes // 2
    src = synth.mixed_bits(36, 0, n + 8, synth.BF16)
    _, ds = to_dev(src)
    fulls, outs = out_buffers([n + 8], _torch_dtype(synth.BF16), GUARD)
    o = off // 2
    A.atom_copy(outs[0][o:], ds[o:], nbytes)
    _sync()
    got = from_dev(outs[0])
    assert_bits_equal(got[o:o + n], src[o:o + n], "copy", nan_by_class=False)
    check_guards(fulls, [n + 8], GUARD)


# --------------------------------------------------------------- AllGather

@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("n", [0, 1, 8, 9, 4096, 100003])
def test_all_gather_zs(A, P, n):
    say(f"AG P={P} n={n}")
    zs = [synth.mixed_bits(37, k, n, synth.BF16) for k in range(P)]
    want = oracle.all_gather(zs)
    dz = [to_dev(z)[1] for z in zs]
    fulls, outs = out_buffers([P * n] * P, _torch_dtype(synth.BF16), GUARD)
    A.all_gather(dz, outs)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"AG out_{j}", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD)


@pytest.mark.parametrize("S", [8 << 10, 64 << 10, (1 << 20) + (48 << 10), 16 << 20])
@pytest.mark.parametrize("chunk", [512 << 10, 1 << 20, 2 << 20])
@pytest.mark.parametrize("slots", [1, 2, 4, 8])
def test_all_gather_snac(A, S, chunk, slots):
    say(f"SNAC AG S={S} chunk={chunk} slots={slots}")
    P = 8
    n = S // 2
    zs = synth.c4_inputs(S, P)
    dz = [to_dev(z)[1] for z in zs]
    outs = [empty_dev(P * n, _torch_dtype(synth.BF16), 0xFFFF) for _ in range(P)]
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk, ring_slots=slots)
    A.all_gather(dz, outs, cfg)
    assert A.atom_sync_status() == A.OK
    import torch
    for j in range(P):
        for k in range(P):
            assert torch.equal(outs[j][k * n:(k + 1) * n].view(torch.int16),
                               dz[k].view(torch.int16)), f"SNAC AG out_{j} block {k}"


@pytest.mark.parametrize("lanes", [64, 128, 512])
@pytest.mark.parametrize("S", [64 << 10, (1 << 20) + (48 << 10)])
@pytest.mark.parametrize("slots", [1, 4])
def test_all_gather_snac_lanes(A, S, slots, lanes):
    """The staged AllGather at every workgroup width other than its default."""
    say(f"SNAC AG S={S} slots={slots} lanes={lanes}")
    P = 8
    n = S // 2
    zs = synth.c4_inputs(S, P)
    dz = [to_dev(z)[1] for z in zs]
    fulls, outs = out_buffers([P * n] * P, _torch_dtype(synth.BF16), GUARD)
    A.all_gather(dz, outs, A.config(flags=A.F_STAGED, chunk_bytes=512 << 10, ring_slots=slots,
                                    lanes=lanes))
    assert A.atom_sync_status() == A.OK
    want = np.concatenate(zs)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want, f"SNAC AG lanes out_{j}", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD)


@pytest.mark.parametrize("wgs", [1, 2, 3, 7, 64])
def test_all_gather_snac_small_grids(A, wgs):
    """Fewer workgroups than ring slots or pieces: ticket order must still
    make progress (one workgroup runs every task in order)."""
    say(f"SNAC AG grid={wgs}")
    P, S = 8, (3 << 20) + (16 << 10)
    n = S // 2
    zs = synth.c4_inputs(S, P)
    dz = [to_dev(z)[1] for z in zs]
    outs = [empty_dev(P * n, _torch_dtype(synth.BF16), 0xFFFF) for _ in range(P)]
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=512 << 10, ring_slots=2, num_wgs=wgs)
    A.all_gather(dz, outs, cfg)
    assert A.atom_sync_status() == A.OK
    want = np.concatenate(zs)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want, f"SNAC small grid out_{j}", nan_by_class=False)


def test_all_gather_snac_repeated(A):
    """Back-to-back staged calls reuse the ring and its flags."""
    P, S = 8, 2 << 20
    n = S // 2
    for rep in range(12):
        say(f"SNAC AG repeat {rep}")
        zs = [synth.draw(40 + rep, k, n, "uniform", synth.BF16) for k in range(P)]
        dz = [to_dev(z)[1] for z in zs]
        outs = [empty_dev(P * n, _torch_dtype(synth.BF16), 0xFFFF) for _ in range(P)]
        cfg = A.config(flags=A.F_STAGED, chunk_bytes=[512 << 10, 1 << 20, 2 << 20][rep % 3],
                       ring_slots=[1, 2, 4, 8][rep % 4])
        A.all_gather(dz, outs, cfg)
        assert A.atom_sync_status() == A.OK
        want = np.concatenate(zs)
        for j in range(P):
            assert_bits_equal(from_dev(outs[j]), want, f"rep {rep} out_{j}", nan_by_class=False)


@pytest.mark.parametrize("lanes", [0, 256])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("n", [8, 40000, 300000])
def test_all_reduce_snac(A, P, n, dtype, lanes):
    """Composed AllReduce through SNAC (Figure 6): the reduced chunk of each
    partition is staged once and fanned out; same bits as the oracle. Both
    workgroup widths: the default (512 lanes) and 256."""
    say(f"SNAC AR P={P} n={n} {dtype} lanes={lanes}")
    xs = [synth.mixed_bits(39, r, P * n, dtype, specials=False) for r in range(P)]
    want = oracle.all_reduce(xs)
    dx = [to_dev(x)[1] for x in xs]
    fulls, outs = out_buffers([P * n] * P, _torch_dtype(dtype), GUARD)
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=3, lanes=lanes)
    A.all_reduce(dx, outs, cfg)
    assert A.atom_sync_status() == A.OK
    for j in range(P):
        _assert_reduced(from_dev(outs[j]), want[j], f"SNAC AR out_{j}")
    check_guards(fulls, [P * n] * P, GUARD)


def test_snac_timeout_is_reported_and_drains(A):
    """Failure handling forced from the host: a 1-microsecond wait bound on a
    one-slot ring shared by 512 workgroups makes producers and consumers give
    up. The kernel must record the timeout, drain every task and exit;
    atom_sync_status reports it once; the next call with the default bound is
    complete and correct."""
    P, S = 8, 4 << 20
    n = S // 2
    zs = synth.c4_inputs(S, P)
    dz = [to_dev(z)[1] for z in zs]
    outs = [empty_dev(P * n, _torch_dtype(synth.BF16), 0xFFFF) for _ in range(P)]
    say("SNAC AG with a 1 us wait bound (expected timeout)")
    # num_wgs: without it the grid follows the ring window (2 workgroups
    # here), which rarely waits long enough to expire a 1 us bound
    A.all_gather(dz, outs, A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=1,
                                    wait_us=1, num_wgs=512))
    assert A.atom_sync_status() == A.ERR_TIMEOUT
    assert A.atom_sync_status() == A.OK            # reported once, then cleared
    say("SNAC AG with the default wait bound after a timeout")
    A.all_gather(dz, outs, A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=1))
    assert A.atom_sync_status() == A.OK
    want = np.concatenate(zs)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want, f"after timeout out_{j}", nan_by_class=False)


# ---------------------------------------------------------------- AllToAll

@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("n", [0, 1, 8, 9, 4096, 30001])
def test_all_to_all(A, P, n):
    say(f"A2A P={P} n={n}")
    xs = [synth.mixed_bits(38, r, P * n, synth.BF16) for r in range(P)]
    want = oracle.all_to_all(xs)
    dx = [to_dev(x)[1] for x in xs]
    fulls, outs = out_buffers([P * n] * P, _torch_dtype(synth.BF16), GUARD)
    A.all_to_all(dx, outs)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"A2A out_{j}", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD)


def _count_cases(P):
    cases = [synth.random_counts(50 + P, P, 37)]
    C = np.zeros((P, P), dtype=np.int64)
    cases.append(C)                                     # nothing moves
    C = np.zeros((P, P), dtype=np.int64)
    C[:, 0] = 11
    cases.append(C)                                     # everything to rank 0
    C = synth.random_counts(60 + P, P, 9, zero_frac=0.0)
    C[P - 1, :] = 0
    cases.append(C)                                     # one silent source
    return cases


@pytest.mark.parametrize("P", [1, 2, 5, 8, 16])
@pytest.mark.parametrize("row", [1, 7, 8, 7168])
def test_all_to_all_v(A, P, row):
    for ci, C in enumerate(_count_cases(P)):
        say(f"A2AV P={P} row={row} case={ci}")
        rows = C.sum(axis=1)
        xs = synth.tagged_rows(P, [int(t) for t in rows], row, seed=ci)
        want = oracle.all_to_all_v(xs, C, row)
        dx = [to_dev(x)[1] if x.size else empty_dev(1, _torch_dtype(synth.BF16)) for x in xs]
        R = C.sum(axis=0)
        sizes = [int(R[j]) * row for j in range(P)]
        fulls, outs = out_buffers(sizes, _torch_dtype(synth.BF16), GUARD)
        A.all_to_all_v(dx, outs, C, row)
        _sync()
        for j in range(P):
            assert_bits_equal(from_dev(outs[j]), want[j], f"A2AV case {ci} out_{j}",
                              nan_by_class=False)
        check_guards(fulls, sizes, GUARD)


# ------------------------------------------------------------- V variants

@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("row", [1, 8, 7168])
def test_v_collectives(A, dtype, row):
    P = 8
    g = synth.rank_rng(70, row)
    cnt = g.integers(0, 9, size=P).astype(np.int64)
    cnt[3] = 0
    T = int(cnt.sum()) * row
    say(f"RSV/AGV row={row} cnt={cnt.tolist()} {dtype}")
    xs = [synth.mixed_bits(71, r, T, dtype, specials=False) for r in range(P)]
    want = oracle.reduce_scatter_v(xs, cnt * row)
    dx = [to_dev(x)[1] for x in xs]
    ys = [empty_dev(max(int(c) * row, 1), _torch_dtype(dtype))[:int(c) * row] for c in cnt]
    A.reduce_scatter_v(dx, ys, cnt, row)
    _sync()
    for k in range(P):
        _assert_reduced(from_dev(ys[k]), want[k], f"RSV y_{k}")
    zs = [synth.mixed_bits(72, k, int(cnt[k]) * row, dtype) for k in range(P)]
    want = oracle.all_gather_v(zs)
    dz = [to_dev(z)[1] if z.size else empty_dev(1, _torch_dtype(dtype)) for z in zs]
    outs = [empty_dev(T, _torch_dtype(dtype)) for _ in range(P)]
    A.all_gather_v(dz, outs, cnt, row)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"AGV out_{j}", nan_by_class=False)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("P", [2, 8, 16])
def test_v_collectives_zipf(A, dtype, P):
    """Figure 16's variable-length workload shape: Zipf(s = 0.125) partition
    sizes, in rows of 8 elements (16-byte partitions for bf16)."""
    T = 8 * 5003 * P
    cnt = synth.zipf_partition(T, P, 0.125, 8) // 8
    say(f"Zipf RSV/AGV P={P} rows={cnt.tolist()} {dtype}")
    xs = [synth.mixed_bits(73, r, T, dtype, specials=False) for r in range(P)]
    want = oracle.reduce_scatter_v(xs, cnt * 8)
    dx = [to_dev(x)[1] for x in xs]
    fulls, ys = out_buffers([int(c) * 8 for c in cnt], _torch_dtype(dtype), GUARD)
    A.reduce_scatter_v(dx, ys, cnt, 8)
    _sync()
    for k in range(P):
        _assert_reduced(from_dev(ys[k]), want[k], f"Zipf RSV y_{k}")
    check_guards(fulls, [int(c) * 8 for c in cnt], GUARD)
    zs = [synth.mixed_bits(74, k, int(cnt[k]) * 8, dtype) for k in range(P)]
    want = oracle.all_gather_v(zs)
    dz = [to_dev(z)[1] for z in zs]
    fulls, outs = out_buffers([T] * P, _torch_dtype(dtype), GUARD)
    A.all_gather_v(dz, outs, cnt, 8)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"Zipf AGV out_{j}", nan_by_class=False)
    check_guards(fulls, [T] * P, GUARD)


@pytest.mark.parametrize("wgs", [1, 3, 8, 13, 0])
def test_xcd_tile_order(A, wgs):
    """The XCD-contiguous tile order (with and without a grid stride) covers
    every tile exactly once: same bits as the oracle for reduce, fan-out and
    exchange."""
    P, n = 8, 40013 * 8
    cfg = A.config(flags=A.F_XCD_ORDER, num_wgs=wgs)
    say(f"XCD order wgs={wgs}")
    xs = [synth.mixed_bits(75, r, P * n, synth.BF16, specials=False) for r in range(P)]
    dx = [to_dev(x)[1] for x in xs]
    ys = [empty_dev(n, _torch_dtype(synth.BF16)) for _ in range(P)]
    A.reduce_scatter(dx, ys, cfg)
    outs = [empty_dev(P * n, _torch_dtype(synth.BF16)) for _ in range(P)]
    A.all_to_all(dx, outs, cfg)
    _sync()
    for k, w in enumerate(oracle.reduce_scatter(xs)):
        _assert_reduced(from_dev(ys[k]), w, f"XCD order RS y_{k}")
    for j, w in enumerate(oracle.all_to_all(xs)):
        assert_bits_equal(from_dev(outs[j]), w, f"XCD order A2A out_{j}", nan_by_class=False)
    A.all_gather(ys, outs, cfg)
    _sync()
    want = np.concatenate([from_dev(y) for y in ys])
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want, f"XCD order AG out_{j}", nan_by_class=False)


@pytest.mark.parametrize("lanes", [64, 128, 256])
@pytest.mark.parametrize("stages", [0, 1, 4])
def test_lanes_and_stages(A, lanes, stages):
    """Every workgroup width and pipeline depth tiles every collective
    exactly: ReduceScatter, fused AllReduce, AllToAllV (ragged counts),
    AllGatherV (Zipf partitions) and the copy, against the oracle, with
    parts that start mid-tile."""
    P, n = 8, 40013 * 8
    cfg = A.config(lanes=lanes, stages=stages)
    say(f"lanes={lanes} stages={stages}")
    xs = [synth.mixed_bits(76, r, P * n, synth.BF16, specials=False) for r in range(P)]
    dx = [to_dev(x)[1] for x in xs]
    ys = [empty_dev(n, _torch_dtype(synth.BF16)) for _ in range(P)]
    A.reduce_scatter(dx, ys, cfg)
    ar = [empty_dev(P * n, _torch_dtype(synth.BF16)) for _ in range(P)]
    A.all_reduce(dx, ar, cfg)
    _sync()
    for k, w in enumerate(oracle.reduce_scatter(xs)):
        _assert_reduced(from_dev(ys[k]), w, f"lanes RS y_{k}")
    want = oracle.all_reduce(xs)
    for j in range(P):
        _assert_reduced(from_dev(ar[j]), want[j], f"lanes AR out_{j}")
    C = synth.random_counts(77, P, 300)
    rows = C.sum(axis=1)
    tx = synth.tagged_rows(P, [int(t) for t in rows], 24)
    dtx = [to_dev(x)[1] if x.size else empty_dev(24, _torch_dtype(synth.BF16)) for x in tx]
    R = C.sum(axis=0)
    outs = [empty_dev(max(int(R[j]), 1) * 24, _torch_dtype(synth.BF16)) for j in range(P)]
    A.all_to_all_v(dtx, outs, C, 24, cfg)
    _sync()
    for j, w in enumerate(oracle.all_to_all_v(tx, C, 24)):
        assert_bits_equal(from_dev(outs[j])[:int(R[j]) * 24], w, f"lanes A2AV out_{j}",
                          nan_by_class=False)
    cnt = synth.zipf_partition(P * 5003 * 8, P, 0.125, 8) // 8
    zs = [synth.mixed_bits(78, k, int(cnt[k]) * 8, synth.BF16) for k in range(P)]
    dz = [to_dev(z)[1] for z in zs]
    tot = int(cnt.sum()) * 8
    ag = [empty_dev(tot, _torch_dtype(synth.BF16)) for _ in range(P)]
    A.all_gather_v(dz, ag, cnt, 8, cfg)
    _sync()
    want = oracle.all_gather_v(zs)
    for j in range(P):
        assert_bits_equal(from_dev(ag[j]), want[j], f"lanes AGV out_{j}", nan_by_class=False)


# ------------------------------------------------------------- side stream

def test_side_stream(A):
    import torch
    P, n = 8, 50000
    xs = [synth.mixed_bits(80, r, P * n, synth.BF16, specials=False) for r in range(P)]
    want = oracle.all_reduce(xs)
    dx = [to_dev(x)[1] for x in xs]
    outs = [empty_dev(P * n, torch.bfloat16) for _ in range(P)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        A.all_reduce(dx, outs, stream=s)
    s.synchronize()
    for j in range(P):
        _assert_reduced(from_dev(outs[j]), want[j], f"side stream out_{j}")


# ------------------------------------------- co-aligned, off 16-byte alignment

@pytest.mark.parametrize("dtype,skew", [(synth.BF16, 1), (synth.BF16, 3), (synth.BF16, 7),
                                        (synth.F32, 1), (synth.F32, 3)])
def test_coaligned_offsets_take_the_vector_path(A, dtype, skew):
    """Every buffer `skew` elements past a 16-byte boundary, partitions of
    16-byte multiples: each part's first elements (the head) are done one by
    one and the rest in 16-byte slots, with a short last slot; every
    collective and the flat copy and reduce match the oracle, and the plan
    reports the vector path."""
    import torch
    P, n = 8, 8 * 4099                     # 16-byte partitions, ragged in tiles
    tdt = _torch_dtype(dtype)
    es = 2 if dtype == synth.BF16 else 4
    say(f"co-aligned skew={skew} {dtype}")

    def dev(a):
        return to_dev(a, pad_before=skew)[1]

    def outs(sizes):
        return out_buffers(sizes, tdt, GUARD + skew)

    xs = [synth.mixed_bits(81, r, P * n, dtype, specials=False) for r in range(P)]
    dx = [dev(x) for x in xs]
    fulls, ys = outs([n] * P)
    st, info = A.atom_plan_query(A.layout(A.PARTITIONED, dx, n), A.layout(A.SHARD, ys, n), A.OP_SUM)
    assert st == A.OK and info.vector_path == 1
    A.reduce_scatter(dx, ys)
    want = oracle.reduce_scatter(xs)
    _sync()
    for k in range(P):
        _assert_reduced(from_dev(ys[k]), want[k], f"RS y_{k}")
    check_guards(fulls, [n] * P, GUARD + skew)
    fulls, ar = outs([P * n] * P)
    A.all_reduce(dx, ar)
    want = oracle.all_reduce(xs)
    _sync()
    for j in range(P):
        _assert_reduced(from_dev(ar[j]), want[j], f"AR out_{j}")
    check_guards(fulls, [P * n] * P, GUARD + skew)
    fulls, a2 = outs([P * n] * P)
    A.all_to_all(dx, a2)
    want = oracle.all_to_all(xs)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(a2[j]), want[j], f"A2A out_{j}", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD + skew)
    zs = [synth.mixed_bits(82, k, n, dtype) for k in range(P)]
    fulls, ag = outs([P * n] * P)
    A.all_gather([dev(z) for z in zs], ag)
    want = oracle.all_gather(zs)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(ag[j]), want[j], f"AG out_{j}", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD + skew)
    # AllToAllV in rows of 16 bytes
    row = 16 // es
    C = synth.random_counts(83, P, 700)
    rows = C.sum(axis=1)
    R = C.sum(axis=0)
    vs = [synth.mixed_bits(84, r, int(rows[r]) * row, dtype) for r in range(P)]
    fulls, av = outs([int(R[j]) * row for j in range(P)])
    A.all_to_all_v([dev(v) if v.size else empty_dev(1, tdt) for v in vs], av, C, row)
    want = oracle.all_to_all_v(vs, C, row)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(av[j]), want[j], f"A2AV out_{j}", nan_by_class=False)
    check_guards(fulls, [int(R[j]) * row for j in range(P)], GUARD + skew)
    # flat copy and flat reduce
    m = 100003 * 8
    src = synth.mixed_bits(85, 0, m, dtype)
    fulls, cp = outs([m])
    A.atom_copy(cp[0], dev(src))
    _sync()
    assert_bits_equal(from_dev(cp[0]), src, "copy", nan_by_class=False)
    check_guards(fulls, [m], GUARD + skew)
    rs = [synth.mixed_bits(86, r, m, dtype, specials=False) for r in range(3)]
    fulls, rd = outs([m])
    A.atom_reduce(rd[0], [dev(x) for x in rs])
    _sync()
    _assert_reduced(from_dev(rd[0]), oracle.reduce(rs), "reduce")
    check_guards(fulls, [m], GUARD + skew)


# ------------------------------------------- blocked fan-out (AllGather(V))

@pytest.mark.parametrize("P", [2, 3, 8, 16])
@pytest.mark.parametrize("skew", [0, 1, 3])
@pytest.mark.parametrize("wgs", [0, 13, 64])
def test_all_gather_blocked_order(A, P, skew, wgs):
    """AllGathers large enough for the blocked fan-out (one output at a
    time per block of tiles): several blocks with a ragged last one, buffers
    skewed off 16-byte alignment by the same amount (element-wise heads in
    the blocked kernel), a caller's grid that is not a multiple of the XCDs
    (grid stride), and the V form with uneven partitions; bit-exact with
    guard canaries."""
    n = (3 << 20) // 2 + 8 * 37          # ~3 MiB partitions, not a whole number of tiles
    say(f"blocked AG P={P} skew={skew} wgs={wgs}")
    tdt = _torch_dtype(synth.BF16)
    zs = [synth.mixed_bits(95, k, n, synth.BF16) for k in range(P)]
    dz = [to_dev(z, pad_before=skew)[1] for z in zs]
    fulls, outs = out_buffers([P * n] * P, tdt, GUARD + skew)
    cfg = A.config(num_wgs=wgs) if wgs else None
    st, info = A.atom_plan_query(A.layout(A.SHARD, dz, n), A.layout(A.GATHERED, outs, n), A.OP_COPY, cfg)
    assert st == A.OK and info.vector_path == 1 and info.lanes == 256
    A.all_gather(dz, outs, cfg)
    _sync()
    want = np.concatenate(zs)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want, f"blocked AG out_{j}", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD + skew)
    # V form: uneven partitions in rows of 8 elements (one of them empty)
    g = synth.rank_rng(96, P)
    cnt = g.integers(0, 2 * n // 8, size=P).astype(np.int64)
    cnt[P // 2] = 0
    T = int(cnt.sum()) * 8
    zv = [synth.mixed_bits(97, k, int(cnt[k]) * 8, synth.BF16) for k in range(P)]
    dv = [to_dev(z, pad_before=skew)[1] if z.size else empty_dev(1, tdt)[:0] for z in zv]
    fulls, outs = out_buffers([T] * P, tdt, GUARD + skew)
    A.all_gather_v(dv, outs, cnt, 8, cfg)
    _sync()
    want = oracle.all_gather_v(zv)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"blocked AGV out_{j}", nan_by_class=False)
    check_guards(fulls, [T] * P, GUARD + skew)


# ------------------------ shifted vector path (sources and outputs disagree)

@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("sk_in,sk_out", [(0, 1), (1, 0), (1, 3), (3, 2)])
def test_shifted_offsets(A, dtype, sk_in, sk_out):
    """Inputs sk_in elements and outputs sk_out elements past a 16-byte
    boundary: each part's sources agree, its destination does not, so every
    collective (and the flat copy and reduce) takes the shifted vector path,
    the 16-byte stores assembled from neighbouring source vectors, with
    element-wise slots at the ends; bit-exact (reductions: also within the
    ulp bar) with guard canaries."""
    P = 8
    es = 2 if dtype == synth.BF16 else 4
    n = 8 * 4099 + (16 // es) // 2            # partitions off 16 bytes too
    tdt = _torch_dtype(dtype)
    say(f"shifted sk_in={sk_in} sk_out={sk_out} {dtype}")

    def dev(a):
        return to_dev(a, pad_before=sk_in)[1] if a.size else empty_dev(1, tdt)[:0]

    def outs(sizes):
        return out_buffers(sizes, tdt, GUARD + sk_out)

    xs = [synth.mixed_bits(87, r, P * n, dtype, specials=False) for r in range(P)]
    dx = [dev(x) for x in xs]
    fulls, ys = outs([n] * P)
    st, info = A.atom_plan_query(A.layout(A.PARTITIONED, dx, n), A.layout(A.SHARD, ys, n), A.OP_SUM)
    assert st == A.OK and info.vector_path == 1 and info.shifted == 1
    A.reduce_scatter(dx, ys)
    want = oracle.reduce_scatter(xs)
    _sync()
    for k in range(P):
        _assert_reduced(from_dev(ys[k]), want[k], f"RS y_{k}")
    check_guards(fulls, [n] * P, GUARD + sk_out)
    fulls, ar = outs([P * n] * P)
    A.all_reduce(dx, ar)
    want = oracle.all_reduce(xs)
    _sync()
    for j in range(P):
        _assert_reduced(from_dev(ar[j]), want[j], f"AR out_{j}")
    check_guards(fulls, [P * n] * P, GUARD + sk_out)
    fulls, a2 = outs([P * n] * P)
    A.all_to_all(dx, a2)
    want = oracle.all_to_all(xs)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(a2[j]), want[j], f"A2A out_{j}", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD + sk_out)
    zs = [synth.mixed_bits(88, k, n, dtype) for k in range(P)]
    fulls, ag = outs([P * n] * P)
    A.all_gather([dev(z) for z in zs], ag)
    want = oracle.all_gather(zs)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(ag[j]), want[j], f"AG out_{j}", nan_by_class=False)
    check_guards(fulls, [P * n] * P, GUARD + sk_out)
    # V forms in single-element rows: segments of any length, some empty,
    # some shorter than 16 bytes
    g = synth.rank_rng(89, P)
    cnt = g.integers(0, 40000, size=P).astype(np.int64)
    cnt[1], cnt[4] = 0, 3
    T = int(cnt.sum())
    xv = [synth.mixed_bits(90, r, T, dtype, specials=False) for r in range(P)]
    fulls, yv = outs([int(c) for c in cnt])
    A.reduce_scatter_v([dev(x) for x in xv], yv, cnt, 1)
    want = oracle.reduce_scatter_v(xv, cnt)
    _sync()
    for k in range(P):
        _assert_reduced(from_dev(yv[k]), want[k], f"RSV y_{k}")
    check_guards(fulls, [int(c) for c in cnt], GUARD + sk_out)
    zv = [synth.mixed_bits(91, k, int(cnt[k]), dtype) for k in range(P)]
    fulls, agv = outs([T] * P)
    A.all_gather_v([dev(z) for z in zv], agv, cnt, 1)
    want = oracle.all_gather_v(zv)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(agv[j]), want[j], f"AGV out_{j}", nan_by_class=False)
    check_guards(fulls, [T] * P, GUARD + sk_out)
    for row in (1, 3, 5):
        C = synth.random_counts(92 + row, P, 900)
        C[2, :] = 0
        C[:, 5] = 1
        rows, R = C.sum(axis=1), C.sum(axis=0)
        vs = [synth.mixed_bits(93, r, int(rows[r]) * row, dtype) for r in range(P)]
        fulls, av = outs([int(R[j]) * row for j in range(P)])
        A.all_to_all_v([dev(v) for v in vs], av, C, row)
        want = oracle.all_to_all_v(vs, C, row)
        _sync()
        for j in range(P):
            assert_bits_equal(from_dev(av[j]), want[j], f"A2AV row={row} out_{j}", nan_by_class=False)
        check_guards(fulls, [int(R[j]) * row for j in range(P)], GUARD + sk_out)
    # flat copy and flat reduce of lengths around the 16-byte boundaries
    for m in (1, 7, 8, 9, 100003):
        src = synth.mixed_bits(94, m, m, dtype)
        fulls, cp = outs([m])
        A.atom_copy(cp[0], dev(src))
        _sync()
        assert_bits_equal(from_dev(cp[0]), src, f"copy m={m}", nan_by_class=False)
        check_guards(fulls, [m], GUARD + sk_out)
        rs = [synth.mixed_bits(95, r, m, dtype, specials=False) for r in range(3)]
        fulls, rd = outs([m])
        A.atom_reduce(rd[0], [dev(x) for x in rs])
        _sync()
        _assert_reduced(from_dev(rd[0]), oracle.reduce(rs), f"reduce m={m}")
        check_guards(fulls, [m], GUARD + sk_out)


@pytest.mark.parametrize("lanes,stages", [(64, 1), (128, 2), (256, 4), (64, 8)])
def test_shifted_launch_shapes(A, lanes, stages):
    """The shifted kernels at every workgroup width and depth (several waves
    per workgroup: the first vector of each wave is loaded by its lane 0),
    on a ReduceScatterV and an AllGatherV of single-element rows."""
    P = 8
    say(f"shifted shapes lanes={lanes} stages={stages}")
    cnt = synth.zipf_partition(8 * 50001, P, 0.125, 1)
    T = int(cnt.sum())
    tdt = _torch_dtype(synth.BF16)
    xs = [synth.mixed_bits(98, r, T, synth.BF16, specials=False) for r in range(P)]
    fulls, ys = out_buffers([int(c) for c in cnt], tdt, GUARD)
    cfg = A.config(lanes=lanes, stages=min(stages, 4))
    A.reduce_scatter_v([to_dev(x)[1] for x in xs], ys, cnt, 1, cfg)
    want = oracle.reduce_scatter_v(xs, cnt)
    _sync()
    for k in range(P):
        _assert_reduced(from_dev(ys[k]), want[k], f"RSV y_{k}")
    check_guards(fulls, [int(c) for c in cnt], GUARD)
    zs = [synth.mixed_bits(99, k, int(cnt[k]), synth.BF16) for k in range(P)]
    fulls, outs = out_buffers([T] * P, tdt, GUARD)
    A.all_gather_v([to_dev(z)[1] for z in zs], outs, cnt, 1, A.config(lanes=lanes, stages=stages))
    want = oracle.all_gather_v(zs)
    _sync()
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"AGV out_{j}", nan_by_class=False)
    check_guards(fulls, [T] * P, GUARD)
