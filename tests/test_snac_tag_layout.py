"""The tagged ring of staged calls that stage each chunk once (CPU only).

A small staged call stages word j (4 bytes) of 16-byte vector v of a piece
in 64-bit pair 256 * (v // 64) + 64 * j + v % 64 of the piece's place
(k_snac.hip, tag_pair), the place of chunk q's piece at byte b starting at
pair (q * chunk + b) / 4. This model replays that arithmetic and checks that
every staged word of a call has a pair of its own, that a piece's pairs stay
inside its place (so two pieces never share a pair), that the whole call
fits the tagged ring (32 MiB: 8 bytes per staged 4), and that each wave-wide
access (64 lanes, one word j) covers 64 adjacent pairs, i.e. whole 128-byte
lines."""

import random

import pytest

TAG_BYTES = 32 << 20


def tag_pair(v, j):
    return ((v >> 6) << 8) + (j << 6) + (v & 63)


def call_pairs(seg_bytes, chunk, piece):
    """{pair: (chunk, piece, v, j)} of every staged word of a call whose
    segments (bytes each) are cut into chunks of `chunk` and pieces of
    `piece` bytes, chunks numbered segment after segment."""
    out, q = {}, 0
    for nbytes in seg_bytes:
        for cbeg in range(0, nbytes, chunk):
            clen = min(chunk, nbytes - cbeg)
            for pbeg in range(0, chunk, piece):
                plen = max(0, min(piece, clen - pbeg))
                base = (q * chunk + pbeg) // 4
                for v in range((plen + 15) // 16):
                    for j in range(4):
                        p = base + tag_pair(v, j)
                        assert p not in out, (q, pbeg, v, j, out.get(p))
                        # inside the piece's own place
                        assert base <= p < base + piece // 4
                        out[p] = (q, pbeg, v, j)
            q += 1
    return out, q


@pytest.mark.parametrize("piece", [8 << 10, 16 << 10, 64 << 10])
def test_every_word_has_a_pair_of_its_own(piece):
    rng = random.Random(piece)
    for _ in range(40):
        nseg = rng.choice([1, 3, 8, 16])
        chunk = piece * rng.choice([1, 2, 4])
        seg = [2 * rng.randrange(0, 3 * chunk // 2) for _ in range(nseg)]
        pairs, q = call_pairs(seg, chunk, piece)
        if 2 * q * chunk <= TAG_BYTES:             # the planner's condition
            assert max(pairs, default=-1) < TAG_BYTES // 8
        assert len(pairs) == sum(4 * ((min(piece, max(0, min(chunk, b - c) - p)) + 15) // 16)
                                 for b in seg for c in range(0, b, chunk)
                                 for p in range(0, chunk, piece))


def test_a_wave_access_covers_whole_lines():
    for w in range(4):                              # waves of a workgroup
        for j in range(4):
            ps = sorted(tag_pair(64 * w + lane, j) for lane in range(64))
            assert ps == list(range(ps[0], ps[0] + 64))
            assert (8 * ps[0]) % 128 == 0           # 512 bytes from a line start
