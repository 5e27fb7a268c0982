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


def stage_and_consume(seg_bytes, chunk, piece, d):
    """A segment whose streams sit d bytes past a 16-byte boundary: each piece
    is staged in the aligned 16-byte vectors that enclose it (vector v holds
    piece bytes [16 v - d, 16 v - d + 16)), in pairs tag_pair(v, j) of a
    place of tag_place pairs, and the consumer writes piece bytes [p0, p1)
    of each vector. Returns {segment byte: (pair, byte in pair)} of every
    byte written, and the largest pair used per place."""
    place = 4 * (piece // 16 + (64 if d else 0))
    written, top = {}, 0
    for q, cbeg in enumerate(range(0, seg_bytes, chunk)):
        clen = min(chunk, seg_bytes - cbeg)
        for i, pbeg in enumerate(range(0, chunk, piece)):
            plen = max(0, min(piece, clen - pbeg))
            base = (q * (chunk // piece) + i) * place
            nv = (d + plen + 15) // 16 if plen > 0 else 0
            for v in range(nv):
                # the enclosing vector's 16 source bytes hold a segment byte
                lo = cbeg + pbeg + 16 * v - d
                assert lo + 16 > 0 and lo < seg_bytes
            for v in range(nv):
                p0 = d if v == 0 else 0
                p1 = min(16, d + plen - 16 * v)
                for b in range(p0, p1):
                    pair = base + tag_pair(v, b // 4)
                    assert base <= pair < base + place
                    top = max(top, pair - base)
                    sb = cbeg + pbeg + 16 * v - d + b     # segment byte
                    assert sb not in written
                    written[sb] = (pair, b % 4)
    return written, top, place


@pytest.mark.parametrize("d", [0, 2, 4, 6, 8, 14])
def test_offset_segments_write_every_byte_once(d):
    rng = random.Random(d)
    for _ in range(25):
        piece = rng.choice([8 << 10, 16 << 10])
        chunk = piece * rng.choice([1, 2, 4])
        seg = 2 * rng.randrange(1, 2 * chunk)           # last chunks short: empty pieces
        written, top, place = stage_and_consume(seg, chunk, piece, d)
        assert sorted(written) == list(range(seg))
        # the enclosing vectors need the extra group only when d > 0
        assert top < place and (d == 0 or top >= 4 * (piece // 16) - 1 or seg < piece)
