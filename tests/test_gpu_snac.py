"""GPU parity of the staged (SNAC) path for every collective, against the CPU
oracle, element by element on the same seeded inputs.

The abstract of "Purlin: Separating Orchestration from the Datapath of
Collectives" makes SNAC the orchestration of every collective, and its
Figure 16 runs the variable-length ones on ordinary (staged) buffers. Each
collective here runs staged with small chunks and rings (so that slots are
reused many times), on 16-byte aligned buffers (the vector path), on
buffers one or three elements off alignment and on partitions whose size
is not a multiple of 16 bytes (the element-wise path), with guard canaries
around every output. Copies and AllToAll(V) must be bit-exact; reductions
within 1 bf16 ulp (fp32: relative 1e-6) and, since both sides add in rank
order and round once, bitwise."""

import numpy as np
import pytest

import oracle
from reduce_atom_03_amd import synth
from tests._helpers import assert_bf16_close, assert_bits_equal, assert_f32_close
from tests.gpu_util import check_guards, empty_dev, from_dev, out_buffers, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu

GUARD = 40


@pytest.fixture(scope="module")
def A():
    require_gpu()
    from reduce_atom_03_amd import atom
    return atom


def _tdt(dtype):
    import torch
    return torch.bfloat16 if dtype == synth.BF16 else torch.float32


def _reduced(got, want, what):
    if want.dtype == np.uint16:
        assert_bf16_close(got, want, 1, what)
    else:
        assert_f32_close(got, want, 1e-6, what)
    assert_bits_equal(got, want, what + " (bitwise)")


def _check_status(A, what):
    st = A.atom_sync_status()
    assert st == A.OK, f"{what}: {A.atom_status_string(st)}"


class Case:
    """Inputs, oracle results and device buffers of one collective call.
    skew: elements each input and output view sits past a 16-byte boundary
    (a list gives one skew per rank); out_skew, when given, the same for
    the outputs alone."""

    def __init__(self, A, coll, P, n, dtype, skew=0, seed=0, out_skew=None):
        self.A, self.coll, self.P, self.dtype = A, coll, P, dtype
        tdt = _tdt(dtype)
        sk = skew if isinstance(skew, list) else [skew] * P
        osk = sk if out_skew is None else (out_skew if isinstance(out_skew, list) else [out_skew] * P)
        self.sk, self.osk = sk, osk

        def dev(a, r):
            if a.size == 0:
                return empty_dev(1, tdt)[:0]
            return to_dev(a, pad_before=sk[r])[1]

        def outs(sizes):
            fulls, views = [], []
            for r, m in enumerate(sizes):
                f, v = out_buffers([m], tdt, GUARD + osk[r])
                fulls.append(f[0])
                views.append(v[0])
            self.fulls, self.sizes = fulls, list(sizes)
            return views

        g = synth.rank_rng(500 + seed, P)
        if coll in ("rsv", "agv"):
            self.cnt = g.integers(0, 2 * n + 1, size=P).astype(np.int64)
            self.cnt[g.integers(0, P)] = 0
            self.row = int(g.integers(1, 5))
        elif coll == "a2av":
            self.cnt = synth.random_counts(600 + seed, P, 2 * n // 3 + 1)
            self.row = int(g.integers(1, 5))
        if coll in ("rs", "ar", "a2a"):
            self.xs = [synth.mixed_bits(510 + seed, r, P * n, dtype, specials=False) for r in range(P)]
            self.dx = [dev(x, r) for r, x in enumerate(self.xs)]
            if coll == "rs":
                self.want = oracle.reduce_scatter(self.xs)
                self.out = outs([n] * P)
                self.lin, self.lout = A.layout(A.PARTITIONED, self.dx, n), A.layout(A.SHARD, self.out, n)
            elif coll == "ar":
                self.want = oracle.all_reduce(self.xs)
                self.out = outs([P * n] * P)
                self.lin, self.lout = A.layout(A.PARTITIONED, self.dx, n), A.layout(A.GATHERED, self.out, n)
            else:
                self.want = oracle.all_to_all(self.xs)
                self.out = outs([P * n] * P)
                self.lin = A.layout(A.PARTITIONED, self.dx, n)
                self.lout = A.layout(A.TRANSPOSED, self.out, n)
        elif coll == "ag":
            self.xs = [synth.mixed_bits(520 + seed, k, n, dtype) for k in range(P)]
            self.dx = [dev(x, r) for r, x in enumerate(self.xs)]
            self.want = oracle.all_gather(self.xs)
            self.out = outs([P * n] * P)
            self.lin, self.lout = A.layout(A.SHARD, self.dx, n), A.layout(A.GATHERED, self.out, n)
        elif coll == "rsv":
            T = int(self.cnt.sum()) * self.row
            self.xs = [synth.mixed_bits(530 + seed, r, T, dtype, specials=False) for r in range(P)]
            self.dx = [dev(x, r) for r, x in enumerate(self.xs)]
            self.want = oracle.reduce_scatter_v(self.xs, self.cnt * self.row)
            self.out = outs([int(c) * self.row for c in self.cnt])
            self.lin = A.layout(A.PARTITIONED, self.dx, 0, self.cnt, self.row)
            self.lout = A.layout(A.SHARD, self.out, 0, None, self.row)
        elif coll == "agv":
            T = int(self.cnt.sum()) * self.row
            self.xs = [synth.mixed_bits(540 + seed, k, int(self.cnt[k]) * self.row, dtype)
                       for k in range(P)]
            self.dx = [dev(x, r) for r, x in enumerate(self.xs)]
            self.want = oracle.all_gather_v(self.xs)
            self.out = outs([T] * P)
            self.lin = A.layout(A.SHARD, self.dx, 0, self.cnt, self.row)
            self.lout = A.layout(A.GATHERED, self.out, 0, None, self.row)
        elif coll == "a2av":
            C = self.cnt
            rows, R = C.sum(axis=1), C.sum(axis=0)
            self.xs = [synth.mixed_bits(550 + seed, r, int(rows[r]) * self.row, dtype) for r in range(P)]
            self.dx = [dev(x, r) for r, x in enumerate(self.xs)]
            self.want = oracle.all_to_all_v(self.xs, C, self.row)
            self.out = outs([int(R[j]) * self.row for j in range(P)])
            self.lin = A.layout(A.PARTITIONED, self.dx, 0, C, self.row)
            self.lout = A.layout(A.TRANSPOSED, self.out, 0, None, self.row)
        self.op = A.OP_SUM if coll in ("rs", "rsv", "ar") else A.OP_COPY

    def run(self, cfg, entry=None):
        (entry or self.A.atom_collective)(self.lin, self.lout, self.op, cfg)

    def plan(self, cfg):
        st, info = self.A.atom_plan_query(self.lin, self.lout, self.op, cfg)
        assert st == self.A.OK
        return info

    def check(self, what):
        for j, w in enumerate(self.want):
            got = from_dev(self.out[j])
            if self.op == self.A.OP_SUM:
                _reduced(got, w, f"{what} out_{j}")
            else:
                assert_bits_equal(got, w, f"{what} out_{j}", nan_by_class=False)
        for f, m, s in zip(self.fulls, self.sizes, self.osk):
            check_guards([f], [m], GUARD + s)


COLLS = ["rs", "rsv", "ag", "agv", "a2a", "a2av", "ar"]


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("coll", COLLS)
@pytest.mark.parametrize("shape", ["aligned", "skew1", "skew3", "ragged", "mixed"])
def test_every_collective_staged(A, coll, shape, dtype):
    """Every collective through SNAC, with 64 KiB chunks in a 3-slot ring and
    16 KiB pieces (every slot reused many times), on aligned buffers, on
    buffers off alignment (skew: every view k elements past a boundary;
    mixed: a different skew per rank) and on partitions whose byte size is
    not a multiple of 16 (ragged)."""
    P = 8
    n = {"ragged": 20003}.get(shape, 20000)
    skew = {"skew1": 1, "skew3": 3, "mixed": [r % 4 for r in range(P)]}.get(shape, 0)
    say(f"staged {coll} {shape} {dtype}")
    c = Case(A, coll, P, n, dtype, skew, seed=COLLS.index(coll))
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=3, piece_bytes=16 << 10)
    info = c.plan(cfg)
    assert info.staged == 1
    if shape == "aligned" and coll not in ("rsv", "agv", "a2av"):
        assert info.vector_path == 1
    c.run(cfg)
    _check_status(A, f"staged {coll} {shape}")
    c.check(f"staged {coll} {shape}")


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("coll", COLLS)
@pytest.mark.parametrize("skews", [(0, 1), (3, 1), (2, 0), (1, "mixed")])
def test_every_collective_staged_shifted(A, coll, skews, dtype):
    """Inputs and outputs at different offsets from 16-byte alignment (in
    elements; mixed: a different output offset per rank): every segment's
    sources agree, so each is staged as vectors at its sources' offset and
    consumed by the shifted path, bit for bit against the oracle; 64 KiB
    chunks in a 3-slot ring with 16 KiB pieces, and the default plan."""
    P = 8
    n = 20000
    sin, sout = skews
    sout = [r % 4 for r in range(P)] if sout == "mixed" else sout
    say(f"staged shifted {coll} in={sin} out={sout} {dtype}")
    c = Case(A, coll, P, n, dtype, sin, seed=70 + COLLS.index(coll), out_skew=sout)
    for cfg in (A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=3, piece_bytes=16 << 10),
                A.config(flags=A.F_STAGED)):
        info = c.plan(cfg)
        assert info.staged == 1 and info.vector_path == 1
        if coll in ("rs", "ag", "ar", "a2a"):
            assert info.shifted == 1
        c.run(cfg)
        _check_status(A, f"staged shifted {coll}")
        c.check(f"staged shifted {coll} in={sin} out={sout}")


@pytest.mark.parametrize("coll", COLLS)
@pytest.mark.parametrize("chunk", [512 << 10, 1 << 20, 2 << 20])
def test_staged_default_plans(A, coll, chunk):
    """Each collective staged with the library's default ring, piece and
    grid at each chunk size of Table 3's range, on messages of several
    chunks per segment."""
    P = 8
    n = 3 * chunk // 2 // 8 + 37 * 8      # bf16: 3/8 chunk per partition plus a tail
    if coll in ("ag",):
        n *= 8
    say(f"staged default {coll} chunk={chunk}")
    c = Case(A, coll, P, n, synth.BF16, 0, seed=10 + COLLS.index(coll))
    c.run(A.config(flags=A.F_STAGED, chunk_bytes=chunk))
    _check_status(A, f"staged default {coll}")
    c.check(f"staged default {coll} chunk={chunk}")


@pytest.mark.parametrize("unit", [8, 1])
@pytest.mark.parametrize("chunk", [512 << 10, 1 << 20, 2 << 20])
def test_staged_zipf_v(A, unit, chunk):
    """Figure 16's workload on ordinary buffers: ReduceScatterV and
    AllGatherV of Zipf(s = 0.125) partitions staged at every chunk size;
    unit 8 keeps partitions at 16-byte multiples (vector path), unit 1
    puts them anywhere (element-wise path)."""
    P = 8
    T = 8 * 300000
    cnt = synth.zipf_partition(T, P, 0.125, unit)
    say(f"staged Zipf RSV/AGV unit={unit} chunk={chunk} cnt={cnt.tolist()}")
    tdt = _tdt(synth.BF16)
    xs = [synth.mixed_bits(560, r, T, synth.BF16, specials=False) for r in range(P)]
    dx = [to_dev(x)[1] for x in xs]
    fulls, ys = out_buffers([int(c) for c in cnt], tdt, GUARD)
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk)
    A.reduce_scatter_v(dx, ys, cnt, 1, cfg)
    _check_status(A, "staged Zipf RSV")
    want = oracle.reduce_scatter_v(xs, cnt)
    for k in range(P):
        _reduced(from_dev(ys[k]), want[k], f"staged Zipf RSV y_{k}")
    check_guards(fulls, [int(c) for c in cnt], GUARD)
    zs = [synth.mixed_bits(561, k, int(cnt[k]), synth.BF16) for k in range(P)]
    dz = [to_dev(z)[1] for z in zs]
    fulls, outs = out_buffers([T] * P, tdt, GUARD)
    A.all_gather_v(dz, outs, cnt, 1, cfg)
    _check_status(A, "staged Zipf AGV")
    want = oracle.all_gather_v(zs)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"staged Zipf AGV out_{j}", nan_by_class=False)
    check_guards(fulls, [T] * P, GUARD)


@pytest.mark.parametrize("P", [1, 2, 3, 16])
@pytest.mark.parametrize("coll", ["rs", "a2a", "a2av", "agv"])
def test_staged_rank_counts(A, P, coll):
    """The staged collectives at other rank counts (A2A: P*P segments)."""
    say(f"staged {coll} P={P}")
    c = Case(A, coll, P, 4099 * 8, synth.F32, 0, seed=20 + P)
    c.run(A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=2))
    _check_status(A, f"staged {coll} P={P}")
    c.check(f"staged {coll} P={P}")


def test_staged_zero_and_empty_segments(A):
    """Counts with zeros everywhere but one pair; and all-zero counts, which
    launch nothing."""
    P = 8
    C = np.zeros((P, P), dtype=np.int64)
    C[5, 2] = 1000
    xs = [synth.mixed_bits(570, r, int(C[r].sum()) * 8, synth.BF16) for r in range(P)]
    dx = [to_dev(x)[1] if x.size else empty_dev(1, _tdt(synth.BF16))[:0] for x in xs]
    R = C.sum(axis=0)
    fulls, outs = out_buffers([int(R[j]) * 8 for j in range(P)], _tdt(synth.BF16), GUARD)
    cfg = A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=1)
    A.all_to_all_v(dx, outs, C, 8, cfg)
    _check_status(A, "staged A2AV one pair")
    want = oracle.all_to_all_v(xs, C, 8)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"one pair out_{j}", nan_by_class=False)
    check_guards(fulls, [int(R[j]) * 8 for j in range(P)], GUARD)
    Z = np.zeros((P, P), dtype=np.int64)
    st, info = A.atom_plan_query(A.layout(A.PARTITIONED, dx, 0, Z, 8),
                                 A.layout(A.TRANSPOSED, outs, 0, None, 8), A.OP_COPY, cfg)
    assert st == A.OK and info.num_wgs == 0
    A.all_to_all_v(dx, outs, Z, 8, cfg)
    _check_status(A, "staged A2AV nothing")


@pytest.mark.parametrize("chunk", [512 << 10, 1 << 20, 2 << 20])
@pytest.mark.parametrize("slots", [1, 2, 4, 8])
def test_staged_hand_off_under_jitter(A, chunk, slots):
    """Stress of the stage/notify/consume hand-off away from its natural
    timing: every notify and every consume of the staged AllGather, the
    staged AllReduce and the staged AllToAllV is delayed by a pseudo-random
    0-40 us (atom_config.jitter_us, a different seed per call), with rings
    of 1-8 slots at each chunk size. Each call must match the oracle bit for
    bit and report no timeout; the test stops at its first mismatch."""
    P = 8
    seeds = [101, 202]
    for coll, n in (("ag", 3 * chunk // 2), ("ar", 3 * chunk // 16), ("a2av", 3 * chunk // 16)):
        c = Case(A, coll, P, n, synth.BF16, 0, seed=30)
        for sd in seeds:
            say(f"jitter {coll} chunk={chunk} slots={slots} seed={sd}")
            cfg = A.config(flags=A.F_STAGED, chunk_bytes=chunk, ring_slots=slots, jitter_us=40,
                           jitter_seed=sd + slots)
            c.run(cfg)
            _check_status(A, f"jitter {coll}")
            c.check(f"jitter {coll} chunk={chunk} slots={slots} seed={sd}")


def test_timeout_is_reported_and_only_its_call_is_incomplete(A):
    """Failure handling forced from the host: a 20 us wait bound against
    producers held up to 3 ms before they notify (the jitter hook) makes
    waits of the first call time out. The kernel records the timeout,
    drains and exits. A second staged call issued before the status check
    must wait normally and be complete and correct; atom_sync_status then
    reports the timeout once."""
    P, S = 8, 1 << 20
    n = S // 2
    zs = synth.c4_inputs(S, P)
    dz = [to_dev(z)[1] for z in zs]
    outs1 = [empty_dev(P * n, _tdt(synth.BF16), 0xFFFF) for _ in range(P)]
    outs2 = [empty_dev(P * n, _tdt(synth.BF16), 0xFFFF) for _ in range(P)]
    say("staged AG forced to time out, then a normal staged AG before the status check")
    A.all_gather(dz, outs1, A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=2,
                                     num_wgs=64, wait_us=20, jitter_us=3000, jitter_seed=5))
    A.all_gather(dz, outs2, A.config(flags=A.F_STAGED, chunk_bytes=64 << 10, ring_slots=2))
    assert A.atom_sync_status() == A.ERR_TIMEOUT
    assert A.atom_sync_status() == A.OK            # reported once, then cleared
    want = np.concatenate(zs)
    for j in range(P):
        assert_bits_equal(from_dev(outs2[j]), want, f"call after the timeout out_{j}",
                          nan_by_class=False)


@pytest.mark.parametrize("counted", [False, True])
@pytest.mark.parametrize("coll,n", [("ag", 4096), ("ar", 512)])
def test_small_call_timeout_leaves_clean_counts(A, coll, n, counted):
    """A small staged call (one workgroup per task, no ticket) clears each
    slot's count word in the task that completes it, and every task counts,
    also one whose wait gave up; on the tagged ring (the default for such a
    call), a consumer that gave up leaves its words with that call's tag,
    which no later call takes. Forced from the host: a 20 us wait bound
    against notifies and consumes held up to 3 ms. The call reports the
    timeout; the same call without the delay, issued right after it and
    before the status check, and then the call on a 2-slot ring (ticket),
    must both be complete and correct."""
    P = 8
    flags = A.F_STAGED | (A.F_COUNTED if counted else 0)
    c = Case(A, coll, P, n, synth.BF16, 0, seed=60)
    info = c.plan(A.config(flags=flags))
    say(f"small {coll} n={n} counted={counted} forced to time out, tasks={info.snac_tasks} "
        f"wgs={info.num_wgs}")
    assert info.num_wgs == info.snac_tasks             # one workgroup per task, no ticket
    assert info.snac_tagged == (0 if counted else 1)
    c.run(A.config(flags=flags, wait_us=20, jitter_us=3000, jitter_seed=11))
    c.run(A.config(flags=flags))
    assert A.atom_sync_status() == A.ERR_TIMEOUT
    assert A.atom_sync_status() == A.OK
    c.check(f"small {coll} after a timed-out call")
    c.run(A.config(flags=flags, ring_slots=2))
    _check_status(A, f"small {coll} ring of 2 after the timeout")
    c.check(f"small {coll} ring of 2 after the timeout")


@pytest.mark.parametrize("counted", [False, True])
@pytest.mark.parametrize("coll,n", [("ag", 4096), ("ar", 512), ("ag", 32768), ("rs", 4096),
                                    ("a2av", 1200), ("rsv", 3000)])
@pytest.mark.parametrize("slots", [1, 2, 64])
def test_small_calls_without_ticket(A, coll, n, slots, counted):
    """Small staged calls (at most 256 tasks, one workgroup each: the default
    64-slot ring) run task blockIdx.x with no ticket, on the tagged ring
    unless ATOM_F_COUNTED asks for the slot counts; rings of 1 and 2 slots
    hold fewer pieces than there are tasks, so the same calls there run
    fewer workgroups on the ticket. Each is checked at natural timing and
    with every notify and consume delayed by a pseudo-random 0-40 us, bit for
    bit against the oracle, twice in a row."""
    P = 8
    c = Case(A, coll, P, n, synth.BF16, 0, seed=40 + slots)
    base = dict(flags=A.F_STAGED | (A.F_COUNTED if counted else 0), ring_slots=slots)
    info = c.plan(A.config(**base))
    say(f"small {coll} n={n} slots={slots} counted={counted} tasks={info.snac_tasks} "
        f"wgs={info.num_wgs} tagged={info.snac_tagged}")
    assert 0 < info.snac_tasks <= 256
    if slots < 64:
        assert info.num_wgs < info.snac_tasks          # the ticket
        assert info.snac_tagged == 0
    elif coll != "a2av":
        assert info.num_wgs == info.snac_tasks         # one workgroup per task, no ticket
    if counted or info.num_wgs < info.snac_tasks:
        assert info.snac_tagged == 0
    elif coll in ("ag", "ar", "rs"):
        assert info.snac_tagged == 1                   # every segment 16-byte aligned
    for jit in (0, 40):
        for rep in range(2):
            cfg = A.config(**base, jitter_us=jit, jitter_seed=7 + rep)
            c.run(cfg)
            _check_status(A, f"small {coll} jitter={jit}")
            c.check(f"small {coll} n={n} slots={slots} jitter={jit} rep={rep}")


def test_tagged_calls_back_to_back(A):
    """Small staged calls on the tagged ring, back to back and interleaved
    with calls that reuse the same workspace through the slot counts (small
    ones with ATOM_F_COUNTED, and a large AllGather that fills the ring with
    other bytes): every call must wait for its own producers, whatever an
    earlier call left in the tagged ring or the ring. Each result is checked
    bit for bit against the oracle; the status is checked at the end."""
    P = 8
    cases = [Case(A, coll, P, n, dt, 0, seed=70 + i)
             for i, (coll, n, dt) in enumerate([("ag", 4096, synth.BF16), ("ar", 512, synth.BF16),
                                                ("rs", 4096, synth.F32), ("a2a", 512, synth.BF16),
                                                ("ag", 65536, synth.BF16), ("rsv", 3000, synth.BF16),
                                                ("ag", 1000, synth.F32), ("ag", 131072, synth.BF16),
                                                ("ar", 65536, synth.F32), ("a2a", 16384, synth.BF16)])]
    big = Case(A, "ag", P, 1 << 20, synth.BF16, 0, seed=79)
    tagged = [c.plan(A.config(flags=A.F_STAGED)).snac_tagged for c in cases]
    say(f"tagged back to back: tagged={tagged}")
    assert sum(tagged) >= 8
    for rep in range(3):
        for i, c in enumerate(cases):
            c.run(A.config(flags=A.F_STAGED))
            c.check(f"rep {rep} case {i} {c.coll} tagged")
            c.run(A.config(flags=A.F_STAGED | A.F_COUNTED))
            c.check(f"rep {rep} case {i} {c.coll} counted")
        big.run(A.config(flags=A.F_STAGED))
        big.check(f"rep {rep} large staged AllGather")
    _check_status(A, "tagged back to back")


@pytest.mark.parametrize("coll,n", [("ag", 524288), ("ag", 1048576), ("ar", 131072), ("rs", 131072),
                                    ("a2a", 65536)])
def test_tagged_medium_calls_under_jitter(A, coll, n):
    """Calls of up to 16 MiB staged on the tagged ring run one workgroup per
    task (here 512-1024 workgroups of 512 lanes, up to twice what the chip holds
    at once): producers never wait, and a consumer waits only for producers
    with smaller workgroup indices. Checked at natural timing and with every
    producer and consumer delayed by a pseudo-random 0-40 us, twice each,
    bit for bit against the oracle."""
    P = 8
    c = Case(A, coll, P, n, synth.BF16, 0, seed=90)
    info = c.plan(A.config(flags=A.F_STAGED))
    say(f"tagged medium {coll} n={n} tasks={info.snac_tasks} wgs={info.num_wgs}")
    assert info.snac_tagged == 1 and info.num_wgs == info.snac_tasks > 256
    for jit in (0, 40):
        for rep in range(2):
            c.run(A.config(flags=A.F_STAGED, jitter_us=jit, jitter_seed=31 + rep))
            _check_status(A, f"tagged medium {coll} jitter={jit}")
            c.check(f"tagged medium {coll} n={n} jitter={jit} rep={rep}")


@pytest.mark.parametrize("counted", [False, True])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
def test_staged_ragged_last_segment(A, dtype, counted):
    """A Zipf-like AllGatherV and ReduceScatterV whose partitions all start
    16-byte aligned but whose last partition ends inside a 16-byte vector
    (and one partition is empty): such a call stays on the vector path, on
    the tagged ring unless ATOM_F_COUNTED asks for the counts, and the
    consumer writes the last partial vector element by element. Bit for bit
    against the oracle, with guard canaries around every output."""
    P = 8
    tdt = _tdt(dtype)
    unit = 16 // (2 if dtype == synth.BF16 else 4)           # elements per 16 bytes
    cnt = np.array([8, 16, 1, 0, 5, 2, 3, 0], np.int64) * unit
    cnt[-1] = 13 if dtype == synth.BF16 else 7
    T = int(cnt.sum())
    cfg = A.config(flags=A.F_STAGED | (A.F_COUNTED if counted else 0))

    def dev(a):
        return empty_dev(1, tdt)[:0] if a.size == 0 else to_dev(a)[1]

    # AllGatherV
    zs = [synth.mixed_bits(950, k, int(cnt[k]), dtype) for k in range(P)]
    dz = [dev(z) for z in zs]
    fulls, outs = out_buffers([T] * P, tdt, GUARD)
    st, info = A.atom_plan_query(A.layout(A.SHARD, dz, 0, cnt, 1), A.layout(A.GATHERED, outs, 0, None, 1),
                                 A.OP_COPY, cfg)
    say(f"ragged AGV dtype={dtype} counted={counted} tagged={info.snac_tagged}")
    assert st == A.OK and info.vector_path == 1 and info.shifted == 0
    assert info.snac_tagged == (0 if counted else 1)
    A.all_gather_v(dz, outs, cnt, 1, cfg)
    _check_status(A, "ragged AGV")
    want = oracle.all_gather_v(zs)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"ragged AGV out_{j}", nan_by_class=False)
    check_guards(fulls, [T] * P, GUARD)
    # ReduceScatterV
    xs = [synth.mixed_bits(960, r, T, dtype, specials=False) for r in range(P)]
    dx = [dev(x) for x in xs]
    fulls, ys = out_buffers([int(c) for c in cnt], tdt, GUARD)
    st, info = A.atom_plan_query(A.layout(A.PARTITIONED, dx, 0, cnt, 1), A.layout(A.SHARD, ys, 0, None, 1),
                                 A.OP_SUM, cfg)
    say(f"ragged RSV dtype={dtype} counted={counted} tagged={info.snac_tagged}")
    assert st == A.OK and info.vector_path == 1 and info.snac_tagged == (0 if counted else 1)
    A.reduce_scatter_v(dx, ys, cnt, 1, cfg)
    _check_status(A, "ragged RSV")
    want = oracle.reduce_scatter_v(xs, cnt)
    for k in range(P):
        _reduced(from_dev(ys[k]), want[k], f"ragged RSV y_{k}")
    check_guards(fulls, [int(c) for c in cnt], GUARD)


@pytest.mark.parametrize("coll,n,dtype,skew", [("ag", 4096, synth.BF16, 1), ("ag", 4096, synth.BF16, 3),
                                               ("ar", 512, synth.BF16, 1), ("rs", 4096, synth.F32, 1),
                                               ("a2a", 2048, synth.BF16, 3), ("ag", 131072, synth.BF16, 5),
                                               ("ar", 131072, synth.F32, 3)])
def test_tagged_calls_off_alignment(A, coll, n, dtype, skew):
    """Every buffer the same few elements off 16-byte alignment: the staged
    call stays on the tagged ring, staging the aligned vectors that enclose
    each piece and writing only the piece's bytes. At natural timing and
    with a 0-40 us jitter, bit for bit against the oracle, guard canaries
    intact."""
    P = 8
    c = Case(A, coll, P, n, dtype, skew, seed=95)
    info = c.plan(A.config(flags=A.F_STAGED))
    say(f"tagged off-alignment {coll} n={n} skew={skew} tagged={info.snac_tagged} tasks={info.snac_tasks}")
    assert info.snac_tagged == 1 and info.vector_path == 1 and info.shifted == 0
    for jit in (0, 40):
        c.run(A.config(flags=A.F_STAGED, jitter_us=jit, jitter_seed=3))
        _check_status(A, f"tagged off-alignment {coll} skew={skew}")
        c.check(f"tagged off-alignment {coll} n={n} skew={skew} jitter={jit}")


@pytest.mark.parametrize("skew", [1, 3])
def test_tagged_offset_uneven_segments(A, skew):
    """An AllGatherV and a ReduceScatterV whose every buffer sits skew
    elements off 16-byte alignment and whose partitions differ in size (in
    multiples of 16 bytes, so every partition starts at that offset): the
    call is tagged, short partitions have empty pieces in their chunk (they
    stage nothing), and every output matches the oracle bit for bit with its
    guard canaries intact."""
    P = 8
    tdt = _tdt(synth.BF16)
    cnt = np.array([32768, 8, 512, 0, 64, 3000, 24, 1000], np.int64) // 8 * 8
    T = int(cnt.sum())
    cfg = A.config(flags=A.F_STAGED)

    def dev(a):
        return empty_dev(1, tdt)[:0] if a.size == 0 else to_dev(a, pad_before=skew)[1]

    zs = [synth.mixed_bits(970 + skew, k, int(cnt[k]), synth.BF16) for k in range(P)]
    dz = [dev(z) for z in zs]
    fulls, outs = out_buffers([T] * P, tdt, GUARD + skew)
    st, info = A.atom_plan_query(A.layout(A.SHARD, dz, 0, cnt, 1), A.layout(A.GATHERED, outs, 0, None, 1),
                                 A.OP_COPY, cfg)
    say(f"tagged offset uneven AGV skew={skew} tagged={info.snac_tagged} chunk={info.chunk_bytes}")
    assert st == A.OK and info.snac_tagged == 1 and info.shifted == 0
    A.all_gather_v(dz, outs, cnt, 1, cfg)
    _check_status(A, "tagged offset uneven AGV")
    want = oracle.all_gather_v(zs)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j]), want[j], f"uneven AGV out_{j}", nan_by_class=False)
    check_guards(fulls, [T] * P, GUARD + skew)
    xs = [synth.mixed_bits(980 + skew, r, T, synth.BF16, specials=False) for r in range(P)]
    dx = [dev(x) for x in xs]
    fulls, ys = out_buffers([int(c) for c in cnt], tdt, GUARD + skew)
    st, info = A.atom_plan_query(A.layout(A.PARTITIONED, dx, 0, cnt, 1), A.layout(A.SHARD, ys, 0, None, 1),
                                 A.OP_SUM, cfg)
    say(f"tagged offset uneven RSV skew={skew} tagged={info.snac_tagged}")
    assert st == A.OK and info.snac_tagged == 1 and info.shifted == 0
    A.reduce_scatter_v(dx, ys, cnt, 1, cfg)
    _check_status(A, "tagged offset uneven RSV")
    want = oracle.reduce_scatter_v(xs, cnt)
    for k in range(P):
        _reduced(from_dev(ys[k]), want[k], f"uneven RSV y_{k}")
    check_guards(fulls, [int(c) for c in cnt], GUARD + skew)
