"""Pins for the oracle's Leech-lattice rules, shells and classes.

* brute force: every same-parity integer vector of squared norm 32 (about
  5.98e8 candidates) is put through the membership rule; exactly 196560 pass,
  the kissing number of the Leech lattice, and the per-pattern tallies equal
  the class counts of the closed-form count;
* the count of every shell m <= 12, summed over its classes, equals the theta
  coefficient (65520/691)(sigma_11(m) - tau(m)), a classical closed form;
* the ball of shells up to 12 has 301 classes and about 1.1e14 points named
  by a 47-bit index (arXiv 2609.02652, section 1, golden fixture).
"""
import json
import os
from itertools import combinations
from multiprocessing import Pool

import numpy as np
import pytest

from oracle import golay, leech

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ brute force

def _patterns(norm, slots=24):
    """Same-parity magnitude multisets (sorted desc) with sum of squares norm."""
    out = []
    for parity in (0, 1):
        vals = [v for v in range(int(norm ** 0.5), -1, -1) if v % 2 == parity]

        def walk(i, left, free, acc):
            if i == len(vals):
                if left == 0 and free == 0:
                    out.append(tuple(acc))
                return
            v = vals[i]
            for c in range(free, -1, -1):
                if c * v * v <= left:
                    walk(i + 1, left - c * v * v, free - c, acc + [v] * c)

        walk(0, norm, slots, [])
    return out


def _placements(pattern):
    """All distinct arrangements of the multiset on 24 positions, as an
    (n, 24) int8 array of magnitudes."""
    distinct = sorted(set(v for v in pattern if v), reverse=True)
    rows = []

    def walk(k, free, row):
        if k == len(distinct):
            rows.append(row.copy())
            return
        v = distinct[k]
        c = pattern.count(v)
        for pos in combinations(free, c):
            for p in pos:
                row[p] = v
            walk(k + 1, [f for f in free if f not in pos], row)
            for p in pos:
                row[p] = 0

    walk(0, list(range(24)), np.zeros(24, dtype=np.int8))
    return np.array(rows, dtype=np.int8)


def _count_chunk(args):
    placements, s0, s1 = args
    nnz = int(np.count_nonzero(placements[0]))
    idx = np.argsort(placements == 0, axis=1, kind="stable")[:, :nnz]
    s = np.arange(s0, s1, dtype=np.int64)
    bits = ((s[:, None] >> np.arange(nnz)) & 1).astype(np.int8)
    signs = np.ones((placements.shape[0], s.size, 24), dtype=np.int8)
    np.put_along_axis(signs, np.broadcast_to(idx[:, None, :], (placements.shape[0], s.size, nnz)),
                      np.broadcast_to(1 - 2 * bits, (placements.shape[0], s.size, nnz)), axis=2)
    x = (placements[:, None, :] * signs).reshape(-1, 24)
    return int(leech.is_leech_batch(x).sum())


def _jobs(pattern, target=1 << 20):
    pl = _placements(pattern)
    nnz = sum(1 for v in pattern if v)
    nsig = 1 << nnz
    if nsig >= target:
        for i in range(pl.shape[0]):
            for s0 in range(0, nsig, target):
                yield (pl[i:i + 1], s0, min(nsig, s0 + target))
    else:
        step = max(1, target // nsig)
        for i in range(0, pl.shape[0], step):
            yield (pl[i:i + step], 0, nsig)


@pytest.mark.slow
def test_shell2_brute_force_kissing_number():
    golay.membership_table()  # build once before forking
    pats = _patterns(32)
    assert sorted(pats) == sorted([
        (4, 4) + (0,) * 22, (4, 2, 2, 2, 2) + (0,) * 19, (2,) * 8 + (0,) * 16, (3,) + (1,) * 23])
    tallies = {}
    with Pool(min(8, os.cpu_count() or 1)) as pool:
        for p in pats:
            tallies[p] = sum(pool.map(_count_chunk, list(_jobs(p))))
    assert sum(tallies.values()) == 196560
    for p, n in tallies.items():
        mult = {v: p.count(v) for v in set(p)}
        assert leech.count_points(mult) == n, p


def test_minimal_vector_examples():
    octad = next(int(w) for w in golay.codewords() if golay.weight(w) == 8)
    x = np.array([2 if (octad >> i) & 1 else 0 for i in range(24)])
    assert leech.is_leech(x)          # (2^8 on an octad, even number of minus signs)
    y = x.copy()
    y[np.nonzero(x)[0][0]] = -2
    assert not leech.is_leech(y)      # one minus sign breaks sum = 0 mod 8
    z = np.zeros(24, dtype=int)
    z[:8] = 2
    if not golay.is_codeword(0xFF):
        assert not leech.is_leech(z)  # 2^8 off an octad
    w = np.ones(24, dtype=int)
    w[0] = -3
    assert leech.is_leech(w)          # (-3, 1^23): 3-mod-4 set is empty
    w[0] = 3
    assert not leech.is_leech(w)


# ------------------------------------------------------------------ theta series

def test_ramanujan_tau_classical_values():
    tau = leech.ramanujan_tau(12)
    assert tau[1:] == [1, -24, 252, -1472, 4830, -6048, -16744, 84480, -113643,
                       -115920, 534612, -370944]
    # Ramanujan's congruence tau(n) = sigma_11(n) mod 691
    for n in range(1, 13):
        assert (tau[n] - leech.sigma(11, n)) % 691 == 0


def test_shell_counts_equal_theta_series():
    assert leech.theta_coefficient(1) == 0
    assert leech.theta_coefficient(2) == 196560
    assert leech.theta_coefficient(3) == 16773120
    for m in range(0, leech.MAX_SHELL + 1):
        assert leech.shell_count(m) == leech.theta_coefficient(m), m


def test_ball_matches_paper():
    facts = json.load(open(os.path.join(GOLDEN, "paper_lattice_facts.json")))
    cl = leech.classes()
    assert sum(1 for c in cl if 2 <= c["m"] <= facts["max_shell"]) == facts["classes_ball12"]
    assert len(cl) == leech.NUM_CLASSES
    n = leech.ball_size(facts["max_shell"])
    assert n == 111043117458001
    assert 2 ** (facts["index_bits"] - 1) < n <= 2 ** facts["index_bits"]
    assert abs(n / facts["ball_points_order"] - 1) < 0.05


def test_class_structure():
    cl = leech.classes()
    assert cl[0]["m"] == 0 and cl[0]["mags"] == (0,)
    keys = [(c["m"], c["key"]) for c in cl]
    assert keys == sorted(keys)
    assert max(len(c["mags"]) for c in cl) == 5        # 3 rank planes suffice
    assert max(c["key"][0] for c in cl) == 13          # |x| <= 13 on the ball
    low = [c for c in cl if 2 <= c["m"] <= 6]
    assert len(low) == 41 and max(len(c["mags"]) for c in low) == 4
    assert max(c["key"][0] for c in low) == 8
    for c in cl[1:]:
        assert sum(v * v for v in c["key"]) == 16 * c["m"]
        assert all(v % 2 == c["parity"] for v in c["key"])


def test_class_of_sampled_points():
    rng = np.random.default_rng(3)
    cl = leech.classes()
    for c in cl[1:40]:
        key = np.array(c["key"])
        for _ in range(3):
            perm = rng.permutation(24)
            assert leech.class_of(key[perm] * rng.choice([-1, 1], 24)) == c["id"]
