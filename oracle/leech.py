"""Leech lattice in integer coordinates, its shells and permutation classes
(oracle; test infrastructure).

Source.  arXiv 2609.02652, section 1 (opening paragraphs and contribution C1):
a 24-weight block is a point of the Leech lattice; the 2-bit rate needs the
union of shells of the ball Lambda24(12), which has 301 coordinate-permutation
classes and about 1.1e14 points named by a 47-bit index.  The lattice rules are
the classical Golay-code construction (the paper's related-work section cites
Conway and Sloane); they are not printed on the pages, so they are written here
from the textbook definition.

Coordinates are integers in the sqrt(8)-scaled frame, where shell m holds the
vectors of squared norm 16*m (shell m <-> norm 2m in the usual frame whose
minimal norm is 4).  Membership, for x in Z^24:
  even type: all x_i even, {i : x_i = 2 mod 4} is a Golay codeword,
             sum(x) = 0 mod 8;
  odd type:  all x_i odd,  {i : x_i = 3 mod 4} is a Golay codeword,
             sum(x) = 4 mod 8.

A coordinate-permutation class is the multiset of |x_i| (reading of "301
coordinate-permutation classes"; the count 301 over shells 2..12 pins it).

Canonical class order (our convention; the pages give none): id 0 is the
origin; the others are sorted ascending by (m, magnitudes sorted descending).

Pins (tests/test_oracle_leech.py): 196560 shell-2 vectors by brute force over
every same-parity candidate of norm 32; per-shell class sums equal the theta
coefficients (65520/691)(sigma_11(m) - tau(m)); 301 classes; ball size in
(2^46, 2^47).
"""
from functools import lru_cache
from math import factorial

import numpy as np

from . import golay

MAX_SHELL = 12
NUM_CLASSES = 302  # 301 classes on shells 2..12 plus the origin


# --------------------------------------------------------------------------
# membership
# --------------------------------------------------------------------------

def _mask_of(bits: np.ndarray) -> np.ndarray:
    """Rows of 24 booleans -> int64 masks with bit i = coordinate i."""
    p = np.packbits(bits, axis=-1, bitorder="little").astype(np.int64)
    return p[:, 0] | (p[:, 1] << 8) | (p[:, 2] << 16)


def is_leech_batch(x: np.ndarray) -> np.ndarray:
    """Membership test for an (n, 24) integer array; returns (n,) bools.
    Residues use two's-complement bit masks: v & 3 == v mod 4 and
    s & 7 == s mod 8 for negative integers too."""
    x = np.asarray(x)
    assert x.ndim == 2 and x.shape[1] == 24 and x.dtype.kind in "iu"
    table = golay.membership_table()
    r4 = x & 3
    s8 = x.sum(axis=1, dtype=np.int64) & 7
    low = (x & 1).astype(bool)
    even = ~low.any(axis=1)
    odd = low.all(axis=1)
    ok_even = even & table[_mask_of(r4 == 2)] & (s8 == 0)
    ok_odd = odd & table[_mask_of(r4 == 3)] & (s8 == 4)
    return ok_even | ok_odd


def is_leech(x) -> bool:
    return bool(is_leech_batch(np.asarray(x).reshape(1, 24))[0])


def shell_of(x) -> int:
    """Shell m of a lattice vector (norm 16 m); raises if the norm is not 16m."""
    n = int(np.sum(np.asarray(x, dtype=np.int64) ** 2))
    if n % 16:
        raise ValueError("norm %d is not a multiple of 16" % n)
    return n // 16


# --------------------------------------------------------------------------
# theta series (classical closed form)
# --------------------------------------------------------------------------

def ramanujan_tau(nmax: int) -> list:
    """tau(0..nmax) from q * prod_{n>=1} (1 - q^n)^24, by truncated power series."""
    poly = [0] * (nmax + 1)
    poly[0] = 1
    for n in range(1, nmax + 1):
        for _ in range(24):
            # multiply by (1 - q^n)
            for k in range(nmax, n - 1, -1):
                poly[k] -= poly[k - n]
    tau = [0] * (nmax + 1)
    for k in range(1, nmax + 1):
        tau[k] = poly[k - 1]
    return tau


def sigma(k: int, n: int) -> int:
    return sum(d ** k for d in range(1, n + 1) if n % d == 0)


def theta_coefficient(m: int) -> int:
    """Number of Leech vectors in shell m: (65520/691)(sigma_11(m) - tau(m))."""
    if m == 0:
        return 1
    tau = ramanujan_tau(m)[m]
    num = 65520 * (sigma(11, m) - tau)
    if num % 691:
        raise ArithmeticError("theta coefficient not integral at m=%d" % m)
    return num // 691


# --------------------------------------------------------------------------
# classes and exact counts
# --------------------------------------------------------------------------

def _multinomial(counts) -> int:
    n = sum(counts)
    out = factorial(n)
    for c in counts:
        out //= factorial(c)
    return out


def _partitions(target: int, slots: int, parity: int, max_val: int):
    """Multisets of `slots` non-negative integers of the given parity with
    sum of squares `target`; yielded as dict value -> count, values <= max_val."""
    vals = [v for v in range(max_val, -1, -1) if v % 2 == parity]

    def rec(i, remaining, left, acc):
        if i == len(vals):
            if remaining == 0 and left == 0:
                yield dict(acc)
            return
        v = vals[i]
        sq = v * v
        if sq == 0:
            if remaining == 0:
                acc[v] = left
                yield {k: c for k, c in acc.items() if c}
                del acc[v]
            return
        cmax = min(left, remaining // sq)
        for c in range(cmax, -1, -1):
            rest = left - c
            rem = remaining - c * sq
            # the smallest value of this parity still available bounds what is left
            smallest = vals[-1] * vals[-1]
            if rem < rest * smallest:
                continue
            if c:
                acc[v] = c
            yield from rec(i + 1, rem, rest, acc)
            if c:
                del acc[v]

    yield from rec(0, target, slots, {})


def count_points(mult: dict) -> int:
    """Number of Leech vectors whose multiset of |x_i| is `mult` (value -> count)."""
    a_w = golay.weight_enumerator()
    values = sorted(mult)
    parity = values[0] % 2
    if any(v % 2 != parity for v in values):
        return 0
    if parity == 0:
        twos = {v: c for v, c in mult.items() if v % 4 == 2}
        zeros = {v: c for v, c in mult.items() if v % 4 == 0}
        w = sum(twos.values())
        if w not in a_w:
            return 0
        nnz = sum(c for v, c in mult.items() if v != 0)
        arr = _multinomial(list(twos.values())) * _multinomial(list(zeros.values()))
        if w > 0:
            signs = 2 ** (nnz - 1)
        else:
            total = sum(v * c for v, c in mult.items())
            signs = 2 ** nnz if total % 8 == 0 else 0
        return a_w[w] * arr * signs
    # odd type: split the multiset into the part on the codeword's support
    items = sorted(mult.items())
    total = 0
    for w, aw in a_w.items():
        def rec(i, left, on):
            nonlocal total
            if i == len(items):
                if left:
                    return
                s = 0
                for (v, c), k in zip(items, on):
                    # on the support x = 3 mod 4, off the support x = 1 mod 4
                    s_on = v if v % 4 == 3 else -v
                    s_off = v if v % 4 == 1 else -v
                    s += k * s_on + (c - k) * s_off
                if s % 8 == 4:
                    total += aw * _multinomial(on) * _multinomial(
                        [c - k for (v, c), k in zip(items, on)])
                return
            v, c = items[i]
            for k in range(0, min(c, left) + 1):
                rec(i + 1, left - k, on + [k])
        rec(0, w, [])
    return total


def _key(mult: dict) -> tuple:
    out = []
    for v in sorted(mult, reverse=True):
        out.extend([v] * mult[v])
    return tuple(out)


@lru_cache(maxsize=1)
def classes() -> tuple:
    """All classes of the ball, canonical order.  Each entry is a dict with
    keys id, m, parity, mags (ascending distinct |x|), key (sorted desc), count."""
    found = [(0, (0,) * 24, {0: 24}, 1)]
    for m in range(1, MAX_SHELL + 1):
        for parity in (0, 1):
            max_val = int((16 * m) ** 0.5)
            for mult in _partitions(16 * m, 24, parity, max_val):
                n = count_points(mult)
                if n > 0:
                    found.append((m, _key(mult), mult, n))
    found.sort(key=lambda t: (t[0], t[1]))
    out = []
    for cid, (m, key, mult, n) in enumerate(found):
        out.append({
            "id": cid,
            "m": m,
            "parity": key[0] % 2,
            "mags": tuple(sorted(mult)),
            "key": key,
            "count": n,
        })
    return tuple(out)


@lru_cache(maxsize=1)
def class_index() -> dict:
    """Map from key (|x| sorted descending) to class id."""
    return {c["key"]: c["id"] for c in classes()}


def class_of(x) -> int:
    key = tuple(sorted((abs(int(v)) for v in x), reverse=True))
    return class_index()[key]


def shell_count(m: int) -> int:
    return sum(c["count"] for c in classes() if c["m"] == m)


def ball_size(max_m: int = MAX_SHELL) -> int:
    return sum(c["count"] for c in classes() if c["m"] <= max_m)
