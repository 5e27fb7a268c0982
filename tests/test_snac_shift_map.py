"""The staged consumer's shifted path (CPU only).

A consumer moves one piece of `size` bytes from the ring, where it starts at
address A (the sources' offset from 16-byte alignment), to destinations that
sit at other offsets (k_snac.hip, consume_shift). Vector v holds ring bytes
[16 v, 16 v + 16); rows of 64 vectors start at vs (chosen so that the first
destination's slots begin a 128-byte line); each lane takes vector v - 1 from
the lane below (lane 0 from the previous row's lane 63, or its own load for a
wave's first row), assembles the destination slot that holds ring bytes
[16 v - d, 16 v - d + 16) with d = (D - A) mod 16, and stores it 16-byte
aligned at D + (16 v - d - A): whole when the slot lies inside the piece,
byte range [p0, p1) otherwise. This model replays that arithmetic on byte
values and checks that every destination byte is written exactly once, with
the ring byte of the same piece offset, nothing outside the piece is
written, the loads stay inside the vectors that hold piece bytes, whole
stores are 16-byte aligned, and each full row of the first destination
starts on a 128-byte line."""

import random

import pytest


def shift_consume(A, size, dests, nthr, U, es):
    """Replay of the kernel's index arithmetic. Returns, per destination,
    {destination address: ring address} of every byte stored, and the
    whole-store addresses."""
    vlo, vhi = A >> 4, (A + size - 1) >> 4
    m0 = dests[0] - A
    M = (m0 - (m0 & 15)) >> 4
    vs = vlo - ((vlo + M) & 7)
    nwave = nthr // 64
    loaded = set()

    def vec(v):
        if vlo <= v <= vhi:
            loaded.add(v)
            return [16 * v + i for i in range(16)]      # ring address of each byte
        return [None] * 16

    written = [dict() for _ in dests]
    whole = [[] for _ in dests]
    rows = [[] for _ in dests]
    for wave in range(nwave):
        w0 = vs + wave * 64 * U
        while w0 <= vhi + 1:
            R = [[vec(w0 + u * 64 + lane) for lane in range(64)] for u in range(U)]
            carry = vec(w0 - 1) if w0 - 1 >= vlo else [None] * 16
            for q, D in enumerate(dests):
                d = (D - A) & 15
                wbase = D + ((w0 - vlo) << 4) - (A & 15) - d
                rows[q].append(wbase)
                for u in range(U):
                    for lane in range(64):
                        if lane > 0:
                            L = R[u][lane - 1]
                        else:
                            L = carry if u == 0 else R[u - 1][63]
                        v = w0 + u * 64 + lane
                        sa = (v << 4) - d
                        lo, hi = A - sa, A + size - sa
                        p0, p1 = max(lo, 0), min(hi, 16)
                        if v > vhi + 1 or p0 >= p1:
                            continue
                        # funnel: the 16 bytes that begin 16 - d bytes into L | R
                        slot = (L + R[u][lane])[16 - d:32 - d]
                        addr = wbase + (u * 64 + lane) * 16
                        if p0 == 0 and p1 == 16:
                            whole[q].append(addr)
                        assert p0 % es == 0 and p1 % es == 0
                        for p in range(p0, p1):
                            assert addr + p not in written[q]
                            written[q][addr + p] = slot[p]
            w0 += nwave * 64 * U
    assert loaded <= set(range(vlo, vhi + 1))
    return written, whole, rows


@pytest.mark.parametrize("es", [2, 4])
@pytest.mark.parametrize("shape", [(512, 2), (256, 2), (64, 1), (128, 4)])
def test_every_byte_once_from_its_ring_byte(es, shape):
    rng = random.Random(1000 * es + shape[0] + shape[1])
    nthr, U = shape
    for _ in range(60):
        size = es * rng.choice([1, 2, 7, 8, 63, 64, 65, 511, 4096, 8191, 16384 + 3, 32768 // es])
        A = (1 << 20) + 16 * rng.randrange(0, 64) + es * rng.randrange(0, 16 // es)
        dests = [(1 << 30) + (q << 24) + 16 * rng.randrange(0, 64) + es * rng.randrange(0, 16 // es)
                 for q in range(rng.choice([1, 8]))]
        written, whole, rows = shift_consume(A, size, dests, nthr, U, es)
        for q, D in enumerate(dests):
            assert sorted(written[q]) == list(range(D, D + size)), (A, size, D)
            for addr, src in written[q].items():
                assert src == A + (addr - D), (A, size, D, addr, src)
            assert all(w % 16 == 0 for w in whole[q])
        # rows of 64 slots start on the first destination's 128-byte lines
        assert all(w % 128 == 0 for w in rows[0])
