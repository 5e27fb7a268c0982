"""Seeded random launch configurations against the oracle.

Each case draws, from its own seed, one collective (ReduceScatter(V),
AllGather(V), AllToAll(V), AllReduce, zero-staging or staged), a rank
count, a length, the dtype, the buffer alignment and a random atom_config
(lanes, stages, num_wgs, flags; chunk, ring slots and piece for staged
calls), and compares every output with the oracle: copies bit-exact,
reductions bitwise (and within 1 bf16 ulp / 1e-6). Guard canaries around
every output must survive. The MoE cases draw routing shapes, row lengths,
buffer offsets and tile settings the same way. The draws are fixed by the seeds, so a failure
names a reproducible case."""

import numpy as np
import pytest

import oracle
from reduce_atom_03_amd import synth
from tests._helpers import assert_bf16_close, assert_bits_equal, assert_f32_close
from tests.gpu_util import check_guards, empty_dev, from_dev, out_buffers, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu

GUARD = 24
KINDS = ["rs", "ar", "ag", "a2a", "rsv", "agv", "a2av",
         "ag_snac", "ar_snac", "rs_snac", "a2a_snac", "rsv_snac", "agv_snac", "a2av_snac"]


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


def _config(A, g, staged):
    kw = {}
    flags = A.F_STAGED if staged else 0
    if g.random() < 0.5:
        kw["lanes"] = int(g.choice([64, 128, 256] + ([512] if staged else [])))
    if g.random() < 0.5:
        kw["stages"] = int(g.choice([1, 2, 4, 8]))
    if g.random() < 0.3:
        kw["num_wgs"] = int(g.integers(1, 3000))
    if staged:
        if g.random() < 0.5:
            kw["chunk_bytes"] = 1 << int(g.integers(16, 22))
        if g.random() < 0.5:
            kw["ring_slots"] = int(g.integers(1, 65))
        if g.random() < 0.3:
            kw["piece_bytes"] = 1 << int(g.integers(14, 17))
    elif g.random() < 0.3:
        flags |= A.F_XCD_ORDER
    if g.random() < 0.3:
        flags |= A.F_NO_NT
    return A.config(flags=flags, **kw), dict(kw, flags=flags)


def _length(g, top):
    return int(np.exp(g.uniform(0, np.log(top)))) if g.random() < 0.9 else int(g.integers(0, 3))


@pytest.mark.parametrize("case", range(280))
def test_random_collective(A, case):
    import torch
    g = np.random.default_rng([913, case])
    kind = KINDS[case % len(KINDS)]
    staged = kind.endswith("_snac")
    kind = kind[:-5] if staged else kind
    P = int(g.integers(1, 17))
    dtype = synth.BF16 if g.random() < 0.6 else synth.F32
    cfg, desc = _config(A, g, staged)
    # inputs and outputs 1-3 elements past a 16-byte boundary (element-aligned
    # only), each on about a third of the cases and drawn apart, so that
    # sources and destinations may sit at different offsets; lengths of any
    # size
    skew = 0 if g.random() < 0.67 else int(g.integers(1, 4))
    oskew = skew if g.random() < 0.5 else (0 if g.random() < 0.5 else int(g.integers(1, 4)))
    seed = 5000 + case
    n = _length(g, 40000)
    say(f"random case {case}: {kind}{' staged' if staged else ''} P={P} n={n} {dtype} "
        f"skew={skew}/{oskew} cfg={desc}")
    tdt = _tdt(dtype)

    def dev(a):
        return to_dev(a, pad_before=skew)[1] if a.size else empty_dev(1, tdt)[:0]

    if kind in ("rs", "ar"):
        xs = [synth.mixed_bits(seed, r, P * n, dtype, specials=False) for r in range(P)]
        dx = [dev(x) for x in xs]
        if kind == "rs":
            want = oracle.reduce_scatter(xs)
            fulls, outs = out_buffers([n] * P, tdt, GUARD + oskew)
            A.reduce_scatter(dx, outs, cfg)
        else:
            want = oracle.all_reduce(xs)
            fulls, outs = out_buffers([P * n] * P, tdt, GUARD + oskew)
            A.all_reduce(dx, outs, cfg)
        assert A.atom_sync_status() == A.OK
        for j in range(P):
            _reduced(from_dev(outs[j]), want[j], f"case {case} out_{j}")
        check_guards(fulls, [o.numel() for o in outs], GUARD + oskew)
    elif kind == "ag":
        zs = [synth.mixed_bits(seed, k, n, dtype) for k in range(P)]
        want = oracle.all_gather(zs)
        fulls, outs = out_buffers([P * n] * P, tdt, GUARD + oskew)
        A.all_gather([dev(z) for z in zs], outs, cfg)
        assert A.atom_sync_status() == A.OK
        for j in range(P):
            assert_bits_equal(from_dev(outs[j]), want[j], f"case {case} out_{j}", nan_by_class=False)
        check_guards(fulls, [P * n] * P, GUARD + oskew)
    elif kind == "a2a":
        xs = [synth.mixed_bits(seed, r, P * n, dtype) for r in range(P)]
        want = oracle.all_to_all(xs)
        fulls, outs = out_buffers([P * n] * P, tdt, GUARD + oskew)
        A.all_to_all([dev(x) for x in xs], outs, cfg)
        torch.cuda.synchronize()
        for j in range(P):
            assert_bits_equal(from_dev(outs[j]), want[j], f"case {case} out_{j}", nan_by_class=False)
        check_guards(fulls, [P * n] * P, GUARD + oskew)
    else:
        row = int(g.choice([1, 3, 8, 24, 64]))
        if kind == "a2av":
            C = synth.random_counts(seed, P, int(g.integers(1, 40)))
            rows = C.sum(axis=1)
            R = C.sum(axis=0)
            xs = [synth.mixed_bits(seed, r, int(rows[r]) * row, dtype) for r in range(P)]
            want = oracle.all_to_all_v(xs, C, row)
            sizes = [int(R[j]) * row for j in range(P)]
            fulls, outs = out_buffers(sizes, tdt, GUARD + oskew)
            A.all_to_all_v([dev(x) for x in xs], outs, C, row, cfg)
            torch.cuda.synchronize()
            for j in range(P):
                assert_bits_equal(from_dev(outs[j]), want[j], f"case {case} out_{j}",
                                  nan_by_class=False)
        else:
            cnt = g.integers(0, max(2, n // max(row, 1) // max(P, 1) + 2), size=P).astype(np.int64)
            T = int(cnt.sum()) * row
            if kind == "rsv":
                xs = [synth.mixed_bits(seed, r, T, dtype, specials=False) for r in range(P)]
                want = oracle.reduce_scatter_v(xs, cnt * row)
                sizes = [int(c) * row for c in cnt]
                fulls, outs = out_buffers(sizes, tdt, GUARD + oskew)
                A.reduce_scatter_v([dev(x) for x in xs], outs, cnt, row, cfg)
                torch.cuda.synchronize()
                for k in range(P):
                    _reduced(from_dev(outs[k]), want[k], f"case {case} y_{k}")
            else:
                zs = [synth.mixed_bits(seed, k, int(cnt[k]) * row, dtype) for k in range(P)]
                want = oracle.all_gather_v(zs)
                sizes = [T] * P
                fulls, outs = out_buffers(sizes, tdt, GUARD + oskew)
                A.all_gather_v([dev(z) for z in zs], outs, cnt, row, cfg)
                torch.cuda.synchronize()
                for j in range(P):
                    assert_bits_equal(from_dev(outs[j]), want[j], f"case {case} out_{j}",
                                      nan_by_class=False)
        check_guards(fulls, sizes, GUARD + oskew)


@pytest.mark.parametrize("case", range(40))
def test_random_moe(A, case):
    """Random routing shape, dtype, capacity cut and tile settings; routing,
    dispatch and combine against the oracle."""
    from tests.test_gpu_moe import _move_case
    g = np.random.default_rng([912, case])
    P = int(g.integers(1, 17))
    E = P * int(g.integers(1, max(2, 1024 // P // 4)))
    k = int(g.integers(1, 17))
    T = int(g.integers(0, 300))
    dt = synth.BF16 if g.random() < 0.6 else synth.F32
    # rows of 16-byte multiples (the 128-bit kernels) and of any length
    # (element-wise), buffers aligned or 1-3 elements off
    H = (int(g.choice([8, 64, 520, 1032, 7, 33, 257])) if dt == synth.BF16
         else int(g.choice([4, 36, 260, 1028, 5, 37])))
    inv = float(g.choice([0.0, 0.05]))
    cut = int(g.integers(0, 4))
    skew_in = 0 if g.random() < 0.7 else int(g.integers(1, 4))
    skew_out = 0 if g.random() < 0.7 else int(g.integers(1, 4))
    cfg = A.config(lanes=int(g.choice([0, 64, 128, 256])), stages=int(g.choice([0, 1, 2, 4, 8])))
    _move_case(A, (6000 + case, P, T, E, k, H, dt, inv, cut), cfg, skew_in, skew_out)
