"""Pins for the oracle's Golay code: facts fixed by classical coding theory."""
from itertools import combinations

import numpy as np

from oracle import golay


def test_size_and_distinct():
    words = golay.codewords()
    assert words.size == 4096
    assert np.unique(words).size == 4096
    assert int(words.max()) < (1 << 24)


def test_weight_enumerator():
    # classical enumerator of the extended binary Golay code
    assert golay.weight_enumerator() == {0: 1, 8: 759, 12: 2576, 16: 759, 24: 1}


def test_linear_and_self_complementary():
    words = set(int(w) for w in golay.codewords())
    rng = np.random.default_rng(1)
    wl = list(words)
    for _ in range(2000):
        a, b = rng.choice(len(wl), 2)
        assert wl[a] ^ wl[b] in words
    assert (1 << 24) - 1 in words


def test_octads_form_steiner_system():
    # every 5-subset of the 24 coordinates lies in exactly one octad: S(5,8,24)
    octads = [int(w) for w in golay.codewords() if golay.weight(w) == 8]
    assert len(octads) == 759
    cover = {}
    for o in octads:
        pos = [i for i in range(24) if (o >> i) & 1]
        for c in combinations(pos, 5):
            cover[c] = cover.get(c, 0) + 1
    assert len(cover) == 42504  # C(24, 5)
    assert set(cover.values()) == {1}


def test_membership_table():
    t = golay.membership_table()
    assert int(t.sum()) == 4096
    for w in golay.codewords()[:64]:
        assert golay.is_codeword(int(w))
    # flipping one bit of a codeword leaves the code (minimum distance 8)
    w = int(golay.codewords()[5])
    for i in range(24):
        assert not golay.is_codeword(w ^ (1 << i))
