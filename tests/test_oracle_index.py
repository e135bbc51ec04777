"""Pins of the 47-bit rank / unrank oracle against things other than itself:
the theta series (shell sizes), an independent construction of the 196,560
minimal vectors (exhaustive round trip on shell 2), the membership test, and
the stated order."""
import bisect
import itertools

import numpy as np
import pytest

from oracle import golay, leech
from oracle import index as oi


def test_total_is_the_ball_size():
    assert oi.total() == 111_043_117_458_001 == leech.ball_size()
    assert 2 ** 46 < oi.total() < 2 ** 47


@pytest.mark.parametrize("m", range(0, 13))
def test_counting_matches_the_theta_series_per_shell(m):
    # points of norm exactly 16 m, summed over the (type, codeword) blocks
    def upto(budget):
        if budget < 0:
            return 0
        n = 0
        for t in (0, 1):
            for mask in golay.codewords():
                nb = golay.weight(int(mask))
                n += oi.completions(t, 24 - nb, nb, budget, t)
        return n
    assert upto(16 * m) - upto(16 * m - 1) == leech.theta_coefficient(m)


def _shell2_vectors():
    """The 196,560 minimal vectors by the classical shapes, built directly:
    (+-4, +-4, 0^22), (+-2^8 on an octad, an even number of minus signs, 0^16)
    and (-3, 1^23) with the signs of a codeword's positions flipped, the 3
    anywhere."""
    out = []
    for i, j in itertools.combinations(range(24), 2):
        for si in (-4, 4):
            for sj in (-4, 4):
                v = [0] * 24
                v[i], v[j] = si, sj
                out.append(v)
    octads = [int(c) for c in golay.codewords() if golay.weight(int(c)) == 8]
    for c in octads:
        pos = [i for i in range(24) if (c >> i) & 1]
        for signs in range(128):
            minus = [(signs >> k) & 1 for k in range(7)]
            minus.append(sum(minus) & 1)  # even number of minus signs
            v = [0] * 24
            for p, mi in zip(pos, minus):
                v[p] = -2 if mi else 2
            out.append(v)
    for p in range(24):
        for c in golay.codewords():
            c = int(c)
            v = [(-1 if (c >> i) & 1 else 1) for i in range(24)]
            v[p] *= -3
            out.append(v)
    return np.array(out, dtype=np.int8)


def test_round_trip_is_exhaustive_on_shell_2():
    pts = _shell2_vectors()
    assert len(pts) == 196_560 == leech.theta_coefficient(2)
    assert np.all(leech.is_leech_batch(pts))
    assert len({p.tobytes() for p in pts}) == 196_560
    ranks = [oi.rank(p) for p in pts]
    assert len(set(ranks)) == 196_560
    assert all(0 <= r < oi.total() for r in ranks)
    # unrank a spread sample back (the whole set takes too long in Python)
    for k in range(0, 196_560, 997):
        assert np.array_equal(oi.unrank(ranks[k]), pts[k])


def test_random_indices_round_trip_and_are_ball_points():
    rng = np.random.default_rng(47)
    idx = [0, 1, oi.total() - 1, int(oi.block_offsets()[4096]), int(oi.block_offsets()[4096]) - 1]
    idx += [int(v) for v in rng.integers(0, oi.total(), 300)]
    for i in idx:
        x = oi.unrank(i)
        assert leech.is_leech(x)
        assert int(np.sum(x.astype(np.int64) ** 2)) <= oi.MAX_NORM
        assert oi.rank(x) == i


def test_order_is_type_then_codeword_then_lexicographic():
    # index 0: the lexicographically smallest even vector with c = 0
    assert list(oi.unrank(0)[:5]) == [-12, -4, -4, -4, 0]
    # the first odd vector starts the second half
    x = oi.unrank(int(oi.block_offsets()[4096]))
    assert np.all(x & 1 == 1)
    # consecutive indices inside a block are lexicographically increasing;
    # across a block boundary the codeword (or the type) changes
    offs = [int(o) for o in oi.block_offsets()]
    rng = np.random.default_rng(3)
    samples = [int(i) for i in rng.integers(0, oi.total() - 1, 50)] + [offs[7] - 1, offs[4096] - 1]
    for i in samples:
        a, b = oi.unrank(i), oi.unrank(i + 1)
        same = bisect.bisect_right(offs, i) == bisect.bisect_right(offs, i + 1)
        if same:
            assert tuple(a.tolist()) < tuple(b.tolist())
        else:
            ca = tuple(((a.astype(int) - (a[0] & 1)) >> 1) & 1)
            cb = tuple(((b.astype(int) - (b[0] & 1)) >> 1) & 1)
            assert ca != cb or (a[0] & 1) != (b[0] & 1)


def test_word_and_shape_gain():
    assert oi.split_word(oi.word(12345, 1)) == (12345, 1)
    assert oi.split_word(oi.word(oi.total() - 1, 0)) == (oi.total() - 1, 0)
    assert oi.word(0, 1) == 1 << 47
    coords = np.zeros((1, 2, 24), dtype=np.int8)
    coords[0, 0, 0], coords[0, 1, 5] = 4, -3
    scale = np.array([np.float16(0.5)]).view(np.uint16)
    tail = np.array([[np.float16(2.0)]]).view(np.uint16)
    w = oi.shape_gain_weights(coords, [[0, 1]], scale, (1.0, 1.25), tail, 49)
    assert w[0, 0] == 2.0 and w[0, 24 + 5] == -3 * 0.5 * 1.25 and w[0, 48] == 2.0
    assert np.count_nonzero(w) == 3
