"""The staged consumer's line-aligned vector order (CPU only).

A consumer moves one piece of `size` bytes; when the piece is a whole number
of 16-byte vectors longer than D, its destination starting D bytes past a
128-byte line, vector v of the loop takes piece byte (16 v - D) mod size
(k_snac.hip, consume_vec),
and lanes whose v lies past the piece store nothing. This model of that
index arithmetic checks the invariant the kernel relies on: every piece byte
is stored exactly once, from the same offset in the ring slot, for every
destination offset, piece size and launch shape; and every wave's stores
after the first fill whole lines."""

import pytest


def consume_map(size, dst_addr, nthr, U):
    D = (dst_addr & 127) if size % 16 == 0 else 0
    if D >= size:
        D = 0
    step = nthr * U * 16
    out = {}
    waves = []
    for b0 in range(0, size, step):
        for u in range(U):
            for w0 in range(0, nthr, 64):
                wave = []
                for lane in range(w0, min(w0 + 64, nthr)):
                    v = b0 + (u * nthr + lane) * 16
                    if v >= size:
                        continue
                    o = v - D + size if v - D < 0 else v - D
                    n = 16 if o + 16 <= size else size - o
                    for k in range(n):
                        assert o + k not in out, (size, dst_addr, o + k)
                        out[o + k] = o + k          # ring byte read == piece byte written
                    wave.append((o, n))
                if wave:
                    waves.append(wave)
    return D, out, waves


@pytest.mark.parametrize("size", [16, 48, 130, 7232, 8192, 8192 - 16, 40000 - 4 * 8192, 65536,
                                  65536 - 32, 196608])
@pytest.mark.parametrize("shape", [(512, 8), (256, 2), (64, 1)])
def test_every_byte_once(size, shape):
    for dst_addr in range(0, 256, 16):
        D, out, waves = consume_map(size, dst_addr, *shape)
        assert sorted(out) == list(range(size))
        if D:
            # every wave but the first stores 64 vectors starting on a line
            # of the destination (dst_addr + o), so it fills whole lines
            for wave in waves[1:]:
                if len(wave) == 64:
                    assert (dst_addr + wave[0][0]) % 128 == 0
