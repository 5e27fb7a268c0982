"""GPU parity of the MoE route, dispatch and combine (Table 2, expert
parallelism) against the CPU oracle, through the C ABI.

* Route: positions, counts and rows received, bit-exact, over shapes that
  cover one and many 256-entry chunks with ragged tails, invalid ids,
  repeated ids, one rank, one expert per rank, 1024 experts, k = 1 and 16,
  and no tokens at all.
* Dispatch: every output row against the oracle (rows no entry lands on keep
  their sentinel), bf16 and fp32, with and without a capacity that drops
  rows; payloads carry NaNs and subnormals and must move bit-exactly.
* Combine: bit-exact against the oracle's binary32 fused multiply-add chain
  (NaN compared by class), bf16 and fp32, signed weights, dropped entries.
* Dispatch and combine with buffers and rows off 16-byte alignment (odd row
  lengths, buffers one to three elements off, rows under 16 bytes; the
  element-wise kernels), with guard elements around every output; and the
  full workload shape one element off.
* The MoE workload at full size (8 ranks x 512 tokens x 7168 bf16, 256
  experts, top-8): route, dispatch and combine against the oracle, and
  combine(dispatch(x)) with weights 1/8 returns x bit for bit (-0 as +0).
"""

import numpy as np
import pytest

import oracle
from reduce_atom_03_amd import synth
from tests._helpers import assert_bits_equal
from tests.gpu_util import empty_dev, from_dev, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    require_gpu()
    from reduce_atom_03_amd import atom
    return atom


def ids_for(seed, P, T, E, k, invalid=0.0, dup=0.0, skew=True):
    """Router-like ids (Gumbel top-k over a Dirichlet popularity), then
    optional invalid ids and repeats planted."""
    if T == 0:
        return [np.zeros(0, dtype=np.int32) for _ in range(P)]
    if skew:
        ids, _ = synth.moe_routing(seed, P, T, E, k)
    else:
        g = np.random.default_rng(seed)
        ids = [np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).reshape(-1)
               .astype(np.int32) for _ in range(P)]
    g = np.random.default_rng(seed + 1)
    for a in ids:
        if dup:
            m = g.random(a.size) < dup
            a[m] = a[np.maximum(np.flatnonzero(m) - 1, 0)]
        if invalid:
            m = g.random(a.size) < invalid
            a[m] = g.choice([-1, E, E + 7, -(2 ** 31), 2 ** 31 - 1], size=int(m.sum()))
    return ids


def route_dev(A, ids, E, k):
    import torch
    dev_ids = [torch.from_numpy(a).to("cuda") if a.size else torch.zeros(1, dtype=torch.int32,
                                                                          device="cuda")
               for a in ids]
    T = ids[0].size // k
    rt = A.moe_alloc_routing(dev_ids, E, k)
    rt.tokens = T
    A.atom_moe_route(rt)
    return rt, dev_ids


def check_route(rt, ids, E, k, what):
    pos, cnt, recv = oracle.moe_route(ids, E, k)
    for r in range(len(ids)):
        got = from_dev(rt.positions_t[r])[:ids[r].size].view(np.int32)
        np.testing.assert_array_equal(got, pos[r], err_msg=f"{what}: positions of rank {r}")
    np.testing.assert_array_equal(from_dev(rt.counts_t).view(np.int32).reshape(cnt.shape), cnt,
                                  err_msg=f"{what}: counts")
    np.testing.assert_array_equal(rt.recv_t.cpu().numpy(), recv, err_msg=f"{what}: rows received")
    return pos, recv


ROUTE_CASES = [  # (seed, P, T, E, k, invalid, dup)
    (1, 8, 512, 256, 8, 0.0, 0.0),
    (2, 8, 700, 64, 3, 0.05, 0.0),      # 2100 entries: 9 chunks, ragged tail
    (3, 4, 37, 8, 4, 0.0, 0.3),         # repeated ids within a token
    (4, 1, 300, 16, 2, 0.1, 0.0),       # one rank
    (5, 8, 129, 8, 1, 0.0, 0.0),        # one expert per rank, k = 1
    (6, 16, 64, 1024, 16, 0.02, 0.0),   # 1024 experts, k = 16, 16 ranks
    (7, 3, 5000, 24, 5, 0.0, 0.0),      # 25000 entries: 98 chunks
    (8, 8, 0, 64, 4, 0.0, 0.0),         # no tokens
    (9, 2, 1, 2, 2, 0.0, 0.0),          # one token
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"seed{c[0]}-P{c[1]}-T{c[2]}-E{c[3]}-k{c[4]}")
def test_route_parity(A, case):
    seed, P, T, E, k, inv, dup = case
    say(f"moe route P={P} T={T} E={E} k={k} invalid={inv} dup={dup}")
    ids = ids_for(seed, P, T, E, k, inv, dup, skew=k < E)
    rt, _ = route_dev(A, ids, E, k)
    check_route(rt, ids, E, k, f"case {case}")
    A.atom_moe_route(rt)                              # idempotent: a second route agrees
    check_route(rt, ids, E, k, f"case {case}, second route")


MOVE_CASES = [  # (seed, P, T, E, k, H, dtype, invalid, cap_cut)
    (11, 8, 64, 32, 4, 7168, synth.BF16, 0.0, 0),
    (12, 4, 33, 8, 3, 72, synth.BF16, 0.1, 0),
    (13, 4, 33, 8, 3, 72, synth.BF16, 0.1, 5),       # capacity drops each rank's last 5 rows
    (14, 3, 50, 6, 2, 36, synth.F32, 0.05, 0),
    (15, 2, 20, 4, 4, 1028, synth.F32, 0.0, 3),
    (16, 8, 40, 64, 16, 256, synth.BF16, 0.0, 0),
    (17, 1, 9, 2, 2, 8, synth.BF16, 0.0, 0),
]


@pytest.mark.parametrize("case", MOVE_CASES, ids=lambda c: f"seed{c[0]}-P{c[1]}-T{c[2]}-k{c[4]}-H{c[5]}-{c[6]}")
def test_dispatch_and_combine_parity(A, case):
    _move_case(A, case, None)


# (lanes, slots per lane): tiles of 1-4 KiB (whole 7168-wide rows are 14 KiB,
# so every shape leaves a short last piece), and every U instantiation
TILE_SHAPES = [(64, 1), (64, 8), (128, 4), (256, 2)]


@pytest.mark.parametrize("shape", TILE_SHAPES, ids=lambda s: f"lanes{s[0]}-U{s[1]}")
@pytest.mark.parametrize("case", [MOVE_CASES[0], MOVE_CASES[1], MOVE_CASES[4]],
                         ids=lambda c: f"seed{c[0]}-H{c[5]}-{c[6]}")
def test_dispatch_and_combine_tile_shapes(A, case, shape):
    _move_case(A, case, A.config(lanes=shape[0], stages=shape[1]))


GUARD = 37          # guard elements after each output (their sentinel must survive)


def _out(n, tdt, fill, skew):
    """n elements at `skew` elements into a buffer with GUARD sentinel
    elements after them: (full buffer, view)."""
    full = empty_dev(skew + max(n, 1) + GUARD, tdt, fill)
    return full, full[skew:skew + max(n, 1)]


def _move_case(A, case, cfg, skew_in=0, skew_out=0):
    import torch
    seed, P, T, E, k, H, dt, inv, cut = case
    say(f"moe dispatch/combine P={P} T={T} E={E} k={k} H={H} {dt} invalid={inv} cut={cut} "
        f"cfg={None if cfg is None else (cfg.lanes, cfg.stages)} skew={skew_in},{skew_out}")
    ids = ids_for(seed, P, T, E, k, inv)
    rt, _ = route_dev(A, ids, E, k)
    pos, recv = check_route(rt, ids, E, k, "route")
    cap = max(int(recv.max()) - cut, 0)
    tdt = torch.bfloat16 if dt == synth.BF16 else torch.float32
    sentinel = 0x7E01 if dt == synth.BF16 else 0x3F812345     # a bf16 NaN; an fp32 number
    xs = [synth.mixed_bits(seed, r, T * H, dt) for r in range(P)]
    x_dev = [to_dev(x, pad_before=skew_in)[1] for x in xs]
    outs = [_out(cap * H, tdt, sentinel, skew_out) for _ in range(P)]
    out_dev = [o[1] for o in outs]
    A.atom_moe_dispatch(rt, x_dev, out_dev, cap, H, cfg=cfg)
    want = oracle.moe_dispatch(xs, ids, pos, E, k, H, cap, fill=sentinel if dt == synth.BF16 else
                               np.uint32(sentinel).view(np.float32))
    for j in range(P):
        full = from_dev(outs[j][0])
        assert_bits_equal(full[skew_out:skew_out + cap * H], want[j], f"dispatch rank {j}",
                          nan_by_class=False)
        guard = np.concatenate([full[:skew_out], full[skew_out + max(cap * H, 1):]])
        assert (guard.view(np.uint16 if dt == synth.BF16 else np.uint32) ==
                (sentinel if dt == synth.BF16 else np.uint32(sentinel))).all(), f"dispatch guard {j}"
    # combine: expert outputs of the dispatch shape, signed weights
    ys = [synth.mixed_bits(seed + 100, j, max(cap, 1) * H, dt) for j in range(P)]
    y_dev = [to_dev(y, pad_before=skew_in)[1] for y in ys]
    g = np.random.default_rng(seed)
    w = [(g.random(T * k, dtype=np.float32) * 3 - 1).astype(np.float32) for _ in range(P)]
    w_dev = [torch.from_numpy(a).to("cuda") if a.size else torch.zeros(1, device="cuda") for a in w]
    outs = [_out(T * H, tdt, sentinel, skew_out) for _ in range(P)]
    o_dev = [o[1] for o in outs]
    A.atom_moe_combine(rt, y_dev, w_dev, o_dev, cap, H, cfg=cfg)
    want = oracle.moe_combine([y[:cap * H] if cap else y[:0] for y in ys], ids, pos, w, E, k, H, cap)
    for r in range(P):
        full = from_dev(outs[r][0])
        assert_bits_equal(full[skew_out:skew_out + T * H], want[r], f"combine rank {r}")
        guard = np.concatenate([full[:skew_out], full[skew_out + max(T * H, 1):]])
        assert (guard.view(np.uint16 if dt == synth.BF16 else np.uint32) ==
                (sentinel if dt == synth.BF16 else np.uint32(sentinel))).all(), f"combine guard {r}"


# Buffers and rows off 16-byte alignment: the element-wise kernels.
ELEM_CASES = [  # (case, skew_in, skew_out)
    ((21, 8, 64, 32, 4, 7167, synth.BF16, 0.0, 0), 0, 0),    # odd row length
    ((11, 8, 64, 32, 4, 7168, synth.BF16, 0.0, 0), 1, 1),    # buffers one element off
    ((11, 8, 64, 32, 4, 7168, synth.BF16, 0.0, 0), 0, 3),    # only the outputs off
    ((22, 4, 33, 8, 3, 37, synth.F32, 0.1, 5), 1, 2),        # fp32, odd rows, drops
    ((23, 3, 50, 6, 2, 5, synth.BF16, 0.05, 0), 2, 0),       # rows shorter than 16 bytes
    ((24, 8, 40, 64, 16, 255, synth.BF16, 0.0, 2), 1, 1),    # k = 16
]


@pytest.mark.parametrize("case,skew_in,skew_out", ELEM_CASES,
                         ids=lambda c: "x" if not isinstance(c, tuple) else f"H{c[5]}-{c[6]}")
def test_dispatch_and_combine_off_alignment(A, case, skew_in, skew_out):
    _move_case(A, case, None, skew_in, skew_out)


def test_moe_workload_one_element_off(A):
    """The full MoE workload shape (8 x 512 x 7168 bf16, 256 experts,
    top-8) with every buffer one element off 16-byte alignment: route,
    dispatch and combine against the oracle."""
    import torch
    P, T, E, k, H = 8, synth.MOE_TOKENS, synth.MOE_EXPERTS, synth.MOE_TOPK, synth.HIDDEN
    say("moe workload, buffers one element off alignment")
    ids, w = synth.moe_routing(6, P, T, E, k)
    xs = synth.moe_inputs()
    rt, _ = route_dev(A, ids, E, k)
    pos, recv = check_route(rt, ids, E, k, "workload route")
    cap = int(recv.max())
    x_dev = [to_dev(x, pad_before=1)[1] for x in xs]
    outs = [_out(cap * H, torch.bfloat16, 0x7E01, 1) for _ in range(P)]
    A.atom_moe_dispatch(rt, x_dev, [o[1] for o in outs], cap, H)
    want = oracle.moe_dispatch(xs, ids, pos, E, k, H, cap, fill=0x7E01)
    for j in range(P):
        assert_bits_equal(from_dev(outs[j][1]), want[j], f"dispatch rank {j}", nan_by_class=False)
    ys = [synth.ranks(60 + j, 1, cap * H, "normal", synth.BF16)[0] for j in range(P)]
    y_dev = [to_dev(y, pad_before=1)[1] for y in ys]
    w_dev = [torch.from_numpy(a).to("cuda") for a in w]
    outs = [_out(T * H, torch.bfloat16, 0, 1) for _ in range(P)]
    A.atom_moe_combine(rt, y_dev, w_dev, [o[1] for o in outs], cap, H)
    want = oracle.moe_combine(ys, ids, pos, w, E, k, H, cap)
    for r in range(P):
        assert_bits_equal(from_dev(outs[r][1]), want[r], f"combine rank {r}")


def test_moe_workload_full(A):
    """8 ranks x 512 tokens x 7168 bf16 N(0,1), 256 experts, top-8 (seed 6)."""
    import torch
    P, T, E, k, H = 8, synth.MOE_TOKENS, synth.MOE_EXPERTS, synth.MOE_TOPK, synth.HIDDEN
    say("moe workload: 8 x 512 x 7168 bf16, E=256, top-8")
    ids, w = synth.moe_routing(6, P, T, E, k)
    xs = synth.moe_inputs()
    rt, _ = route_dev(A, ids, E, k)
    pos, recv = check_route(rt, ids, E, k, "workload route")
    cap = int(recv.max())
    x_dev = [to_dev(x)[1] for x in xs]
    out_dev = [empty_dev(cap * H, torch.bfloat16, 0) for _ in range(P)]
    A.atom_moe_dispatch(rt, x_dev, out_dev, cap, H)
    want = oracle.moe_dispatch(xs, ids, pos, E, k, H, cap)
    for j in range(P):
        assert_bits_equal(from_dev(out_dev[j]), want[j], f"workload dispatch rank {j}")
    # combine of stand-in expert outputs (N(0,1) rows in dispatch layout)
    # with the router's gate weights
    ys = [synth.ranks(60 + j, 1, cap * H, "normal", synth.BF16)[0] for j in range(P)]
    y_dev = [to_dev(y)[1] for y in ys]
    w_dev = [torch.from_numpy(a).to("cuda") for a in w]
    o_dev = [empty_dev(T * H, torch.bfloat16, 0) for _ in range(P)]
    A.atom_moe_combine(rt, y_dev, w_dev, o_dev, cap, H)
    want = oracle.moe_combine(ys, ids, pos, w, E, k, H, cap)
    for r in range(P):
        assert_bits_equal(from_dev(o_dev[r]), want[r], f"workload combine rank {r}")
    # identity experts, weights 1/8: every token comes back exactly, except
    # that -0 comes back as +0 (the sum starts from +0)
    uni = [torch.full((T * k,), 1.0 / k, dtype=torch.float32, device="cuda") for _ in range(P)]
    A.atom_moe_combine(rt, out_dev, uni, o_dev, cap, H)
    for r in range(P):
        want = np.where(xs[r] == 0x8000, 0, xs[r]).astype(np.uint16)
        assert_bits_equal(from_dev(o_dev[r]), want, f"round trip {r}")


def test_moe_many_tokens_sampled(A):
    """4096 tokens per rank (32768 entries: 128 chunks), 1024-wide rows:
    route in full, dispatch checked on every row against its token."""
    import torch
    P, T, E, k, H = 8, 4096, 256, 8, 1024
    say("moe many tokens: 8 x 4096 tokens, E=256, top-8, H=1024")
    ids, w = synth.moe_routing(9, P, T, E, k)
    rt, _ = route_dev(A, ids, E, k)
    pos, recv = check_route(rt, ids, E, k, "route")
    cap = int(recv.max())
    # tokens identify themselves: element 0 = rank, element 1 = token
    xs = synth.tagged_rows(P, [T] * P, H)
    x_dev = [to_dev(x)[1] for x in xs]
    out_dev = [empty_dev(cap * H, torch.bfloat16, 0xFFFF) for _ in range(P)]
    A.atom_moe_dispatch(rt, x_dev, out_dev, cap, H)
    per = E // P
    all_rows = np.stack([x.reshape(T, H) for x in xs])
    for j in range(P):
        o = from_dev(out_dev[j]).reshape(cap, H)
        src_r, src_t = np.full(cap, -1), np.full(cap, -1)
        for r in range(P):
            e = ids[r]
            sel = (e >= j * per) & (e < (j + 1) * per)
            src_r[pos[r][sel]] = r
            src_t[pos[r][sel]] = np.flatnonzero(sel) // k
        assert (src_r[:int(recv[j])] >= 0).all()
        rows = all_rows[src_r[:int(recv[j])], src_t[:int(recv[j])]]
        assert_bits_equal(o[:int(recv[j])], rows, f"rank {j}")
        assert (o[int(recv[j]):] == 0xFFFF).all()


def test_moe_maximum_entries_by_properties(A):
    """The largest routing the ABI takes: 16 ranks x 65536 tokens x top-16
    (2**20 entries per rank) over 1024 experts. The oracle's loops are too
    slow here, so the layout is checked by what defines it, vectorized: per
    destination rank the positions are a permutation of 0..recv-1 whose
    order is (expert, source rank, entry); counts are the histogram of the
    ids; and every dispatched 16-byte row carries its own (rank, token)."""
    import torch
    P, T, E, k, H = 16, 65536, 1024, 16, 8
    say("moe maximum: 16 ranks x 65536 tokens x top-16, E=1024")
    g = np.random.default_rng(77)
    ids = [g.integers(0, E, size=T * k, dtype=np.int64).astype(np.int32) for _ in range(P)]
    ids[3][::997] = -5                                  # some entries route nowhere
    rt, _ = route_dev(A, ids, E, k)
    torch.cuda.synchronize()
    pos = [rt.positions_t[r].cpu().numpy() for r in range(P)]
    cnt = rt.counts_t.cpu().numpy().reshape(P, E)
    recv = rt.recv_t.cpu().numpy()
    per = E // P
    for r in range(P):
        valid = (ids[r] >= 0) & (ids[r] < E)
        assert (pos[r][~valid] == -1).all()
        np.testing.assert_array_equal(cnt[r], np.bincount(ids[r][valid], minlength=E))
    ent = np.arange(T * k, dtype=np.int64)
    for j in range(P):
        e_all, key_all, p_all = [], [], []
        for r in range(P):
            sel = (ids[r] >= j * per) & (ids[r] < (j + 1) * per)
            e = ids[r][sel].astype(np.int64)
            key_all.append((e << 24) | (r << 20) | ent[sel])     # (expert, rank, entry)
            p_all.append(pos[r][sel].astype(np.int64))
        key = np.concatenate(key_all)
        p = np.concatenate(p_all)
        assert recv[j] == key.size
        order = np.argsort(p, kind="stable")
        np.testing.assert_array_equal(p[order], np.arange(key.size))
        assert (np.diff(key[order]) > 0).all(), f"rank {j}: rows out of (expert, source, entry) order"
    # dispatch of self-identifying rows (element 0 = rank, element 1 = token)
    cap = int(recv.max())
    xs = synth.tagged_rows(P, [T] * P, H)
    x_dev = [to_dev(x)[1] for x in xs]
    out_dev = [empty_dev(cap * H, torch.bfloat16, 0xFFFF) for _ in range(P)]
    A.atom_moe_dispatch(rt, x_dev, out_dev, cap, H)
    outs = [from_dev(o).reshape(cap, H) for o in out_dev]
    for r in range(P):
        valid = pos[r] >= 0
        j = ids[r][valid] // per
        for jj in range(P):
            m = j == jj
            rows = outs[jj][pos[r][valid][m]]
            assert (rows[:, 0] == r).all(), f"source {r} -> rank {jj}: wrong rank tag"
            np.testing.assert_array_equal(rows[:, 1], (ent[valid][m] // k) & 0xFFFF)
