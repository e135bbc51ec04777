"""47-bit rank / unrank of the Leech-lattice ball and shape-gain dequantisation
(oracle; test infrastructure).

Sources.  arXiv 2609.02652 serves the quantised weights of the source method
as one 48-bit word per 24-weight block, "47-bit indices plus one gain bit",
produced by a GPTQ loop with shape-gain coding (quality protocol paragraph and
the published-results paragraph: 48 bits per 24-weight block), and unfolds
them into its GPU layouts at load time (the validity-envelope paragraph).
The index runs over the points of Lambda24 on shells m <= 12 (the 301-class
ball of section 1), 111,043,117,458,001 points, between 2^46 and 2^47.

Reading (the pages fix neither the enumeration order nor the gain levels):
  * A lattice vector in the sqrt(8)-scaled frame is x = r + 4 z with
    r = 2 c (even type) or r = 1 + 2 c (odd type), c an extended Golay
    codeword (0/1 per coordinate) and z an integer vector with sum(z) even
    (even type) or odd (odd type).  This is the membership rule written as a
    decomposition: x mod 4 gives r, and the sum condition mod 8 becomes the
    parity of sum(z).
  * Order: even type before odd type; inside a type, codewords in the order
    of their 12-bit message (oracle.golay.codewords()); inside a codeword,
    vectors in lexicographic order of (x_0, x_1, ..., x_23) with each
    coordinate's values ascending.  The index of a vector is the number of
    ball points before it in that order.
  * Word: bits 0..46 the index, bit 47 the gain bit.
  * Shape-gain: the dequantised block is w = s_r * gamma[g] * x with the row
    scale s_r and two gain levels gamma[0], gamma[1] given with the matrix
    (parity unpinned for the gain values: the pages give none).

Counting: F(nA, nB, budget, parity) = number of ways to fill nA coordinates
with c = 0 and nB with c = 1 so that the norm stays within the budget and the
parities of their z add up to `parity`; written as the plain recursion over
one coordinate at a time, memoised.  Pinned in tests/test_oracle_index.py:
the total equals the ball size from the theta series, the round trip is
exhaustive on shell 2, and every unranked vector passes the membership test.
"""
from functools import lru_cache

import numpy as np

from . import golay, leech

MAX_NORM = 16 * leech.MAX_SHELL  # 192: shells m <= 12
INDEX_BITS = 47
GAIN_BIT = 47


def residue(t: int, ci: int) -> int:
    return 2 * ci if t == 0 else 1 + 2 * ci


def values(t: int, ci: int) -> tuple:
    """Coordinate values v = r + 4 z with v^2 <= MAX_NORM, ascending."""
    r = residue(t, ci)
    out = []
    v = r
    while v * v <= MAX_NORM:
        v -= 4
    v += 4
    while v * v <= MAX_NORM:
        out.append(v)
        v += 4
    return tuple(out)


def zpar(t: int, ci: int, v: int) -> int:
    return ((v - residue(t, ci)) // 4) & 1


@lru_cache(maxsize=None)
def completions(t: int, n_a: int, n_b: int, budget: int, parity: int) -> int:
    """Ways to give n_a coordinates with c = 0 and n_b with c = 1 values of
    type t with sum of squares <= budget and sum of z parities = parity."""
    if budget < 0:
        return 0
    if n_a == 0 and n_b == 0:
        return 1 if parity == 0 else 0
    ci = 0 if n_a > 0 else 1
    total = 0
    for v in values(t, ci):
        if v * v > budget:
            continue
        total += completions(t, n_a - (1 - ci), n_b - ci, budget - v * v,
                             parity ^ zpar(t, ci, v))
    return total


def _bits(mask: int) -> list:
    return [(int(mask) >> i) & 1 for i in range(24)]


def _type_parity(t: int) -> int:
    return t  # sum(z) even for the even type, odd for the odd type


def block_size(t: int, mask: int) -> int:
    """Ball points of type t with residue pattern given by codeword `mask`."""
    nb = golay.weight(mask)
    return completions(t, 24 - nb, nb, MAX_NORM, _type_parity(t))


@lru_cache(maxsize=1)
def block_offsets() -> np.ndarray:
    """Start index of each (type, codeword) block: 8193 Python ints (object)."""
    offs = [0]
    for t in (0, 1):
        for mask in golay.codewords():
            offs.append(offs[-1] + block_size(t, int(mask)))
    return np.array(offs, dtype=object)


def total() -> int:
    return int(block_offsets()[-1])


def _suffix_counts(c: list) -> list:
    """(nA, nB) of coordinates i+1 .. 23, for each i."""
    out = []
    for i in range(24):
        rest = c[i + 1:]
        nb = sum(rest)
        out.append((len(rest) - nb, nb))
    return out


def rank(x) -> int:
    """Index of a ball point (int sequence of 24, Leech, norm <= 192)."""
    x = [int(v) for v in x]
    assert leech.is_leech(np.array(x)) and sum(v * v for v in x) <= MAX_NORM
    t = x[0] & 1
    c = [((v - t) >> 1) & 1 for v in x]  # x = t + 2c (mod 4)
    mask = sum(b << i for i, b in enumerate(c))
    msg = int(np.nonzero(golay.codewords() == mask)[0][0])
    idx = int(block_offsets()[t * 4096 + msg])
    budget, parity = MAX_NORM, _type_parity(t)
    rest = _suffix_counts(c)
    for i in range(24):
        na, nb = rest[i]
        for v in values(t, c[i]):
            if v == x[i]:
                break
            if v * v <= budget:
                idx += completions(t, na, nb, budget - v * v, parity ^ zpar(t, c[i], v))
        budget -= x[i] * x[i]
        parity ^= zpar(t, c[i], x[i])
    return idx


def unrank(idx: int) -> np.ndarray:
    """The ball point with index idx (0 <= idx < total())."""
    idx = int(idx)
    offs = block_offsets()
    assert 0 <= idx < total()
    blk = int(np.searchsorted(offs.astype(float), float(idx), side="right")) - 1
    # float search is approximate at 1e14: settle the block exactly
    while offs[blk] > idx:
        blk -= 1
    while offs[blk + 1] <= idx:
        blk += 1
    t, msg = divmod(blk, 4096)
    c = _bits(golay.codewords()[msg])
    idx -= int(offs[blk])
    budget, parity = MAX_NORM, _type_parity(t)
    rest = _suffix_counts(c)
    x = []
    for i in range(24):
        na, nb = rest[i]
        for v in values(t, c[i]):
            if v * v > budget:
                continue
            n = completions(t, na, nb, budget - v * v, parity ^ zpar(t, c[i], v))
            if idx < n:
                break
            idx -= n
        else:
            raise AssertionError("index past the block")
        x.append(v)
        budget -= v * v
        parity ^= zpar(t, c[i], v)
    return np.array(x, dtype=np.int8)


def word(idx: int, gain: int) -> int:
    assert 0 <= idx < (1 << INDEX_BITS) and gain in (0, 1)
    return int(idx) | (int(gain) << GAIN_BIT)


def split_word(w: int) -> tuple:
    w = int(w)
    return w & ((1 << INDEX_BITS) - 1), (w >> GAIN_BIT) & 1


def shape_gain_weights(coords, gain_bits, scale_bits, gains, tail_bits, cols: int) -> np.ndarray:
    """f64 W of a matrix of blocks: w = s_r * gamma[g] * x, tail unscaled.
    coords int8 [R][nb][24], gain_bits [R][nb] in {0, 1}, gains (g0, g1)."""
    from .gemv import f16, leech_weights
    coords = np.asarray(coords)
    rows, nb = coords.shape[0], coords.shape[1]
    g = np.asarray(gains, dtype=np.float64)[np.asarray(gain_bits, dtype=np.int64)]
    w = leech_weights(coords, scale_bits, tail_bits, cols)
    w[:, : 24 * nb] *= np.repeat(g.reshape(rows, nb), 24, axis=1)
    return w
