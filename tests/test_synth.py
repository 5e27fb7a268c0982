"""The seeded input generators: determinism, shapes and the Zipf partition."""

import numpy as np
import pytest

from reduce_atom_03_amd import synth


def test_draws_are_deterministic_and_rank_distinct():
    a = synth.draw(2, 0, 1000, "normal", synth.BF16)
    b = synth.draw(2, 0, 1000, "normal", synth.BF16)
    c = synth.draw(2, 1, 1000, "normal", synth.BF16)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    threaded = synth.ranks(2, 4, 1 << 20, "normal", synth.F32, threads=4)
    serial = synth.ranks(2, 4, 1 << 20, "normal", synth.F32, threads=1)
    for x, y in zip(threaded, serial):
        assert np.array_equal(x, y)


def test_distributions():
    u = synth.draw(1, 0, 1 << 16, "uniform", synth.F32)
    assert u.min() >= -1 and u.max() <= 1 and abs(u.mean()) < 0.02
    g = synth.draw(5, 0, 1 << 16, "normal", synth.F32, scale=0.02)
    assert abs(g.std() - 0.02) < 0.001


@pytest.mark.parametrize("P", [1, 2, 5, 8, 16])
@pytest.mark.parametrize("unit", [1, 8, 7168])
def test_zipf_partition(P, unit):
    total = 1000 * unit * P
    sizes = synth.zipf_partition(total, P, 0.125, unit)
    assert sizes.sum() == total and (sizes % unit == 0).all() and (sizes >= 0).all()
    # non-increasing, and within one unit of the exact Zipf shares
    assert (np.diff(sizes) <= unit).all()
    w = np.arange(1, P + 1) ** -0.125
    assert np.all(np.abs(sizes / unit - total / unit * w / w.sum()) < 1.0 + 1e-9)
    assert np.array_equal(synth.zipf_partition(total, P, 0.0, unit), np.full(P, total // P))
