"""Seeded synthetic inputs for every workload (shared by tests and bench).

This module only draws inputs: integer Leech-lattice blocks, fp16 scales,
tails, coefficients, trellis bit streams and tables, and fp16 activations.  It
holds none of the dequantize or matvec arithmetic, and it imports neither the
oracle nor the HIP library (it carries its own Golay code and its own class
counts, used only to sample uniformly).

Every array has its own stream:
    numpy.random.default_rng(SeedSequence([0, cfg, arr, rows, cols]))
with arr numbered coords=0, scales=1, x=2, tail/coeffs/bits=3, table=4,
zero-mask=5, dense control W=6; the weight stack of a model uses
SeedSequence([0, 5, layer, matrix, arr, rows, cols]).  Adding batch columns to
x never changes W.

Workloads (they stand in for the Qwen3 projections of the pages; no dataset
or checkpoint is involved):
  cfg 1  Leech 1536x1536: shell m uniform on {2, 3}, then a uniform point of
         that shell; each block independently the origin with probability 0.02.
  cfg 2  BPDQ 4096x4096, group 256: Bernoulli(0.5) bits, coefficients fp16
         N(0, 0.02^2); dense fp16 control W ~ fp16 N(0, 0.02^2).
  cfg 3  Leech 4096x4096 and 12288x4096: m in 2..6 with P(m) proportional to
         2^-m, uniform within the shell; tail fp16 N(0, 0.02^2).
  cfg 4  bitshift trellis 4096x12288: Bernoulli(0.5) bits, a 65536-entry fp16
         N(0, 1) table, per-row scale; and the Leech matrix of the same shape
         drawn like cfg 3.
  cfg 5  a Qwen3-8B-shaped stack of 36 layers x {q, k, v, o, gate, up, down}
         drawn like cfg 3.
Scales are fp16(|N(0,1)| * 0.02); x is fp16 N(0,1); fp16 rounding is
round-to-nearest-even.
"""
from functools import lru_cache
from math import factorial

import numpy as np

ARR_COORDS, ARR_SCALE, ARR_X, ARR_AUX, ARR_TABLE, ARR_ZERO, ARR_DENSE = range(7)

QWEN3_8B_MATRICES = (
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288),
)
QWEN3_8B_LAYERS = 36


def rng_for(*key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def fp16_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------
# Golay code and class counts, for uniform sampling only
# --------------------------------------------------------------------------

@lru_cache(maxsize=1)
def _golay_words() -> np.ndarray:
    # cyclic [23,12] code, g(x) = 1 + x^2 + x^4 + x^5 + x^6 + x^10 + x^11,
    # extended by an overall parity bit at position 23
    g = sum(1 << e for e in (0, 2, 4, 5, 6, 10, 11))
    gens = []
    for shift in range(12):
        v = g << shift
        gens.append(v | ((bin(v).count("1") % 2) << 23))
    words = np.zeros(1 << 12, dtype=np.int64)
    for msg in range(1, 1 << 12):
        low = msg & -msg
        words[msg] = words[msg ^ low] ^ gens[low.bit_length() - 1]
    return words


@lru_cache(maxsize=1)
def _golay_by_weight() -> dict:
    words = _golay_words()
    pc = np.array([bin(int(w)).count("1") for w in words])
    return {int(w): words[pc == w] for w in np.unique(pc)}


@lru_cache(maxsize=1)
def _golay_bits() -> np.ndarray:
    words = _golay_words()
    return ((words[:, None] >> np.arange(24)) & 1).astype(np.int8)


def _perms(counts) -> int:
    out = factorial(sum(counts))
    for c in counts:
        out //= factorial(c)
    return out


def _multisets(norm: int, parity: int):
    """Same-parity multisets of 24 magnitudes with sum of squares `norm`,
    as tuples sorted descending."""
    top = int(norm ** 0.5)
    vals = [v for v in range(top, -1, -1) if v % 2 == parity]
    out = []

    def walk(i, left, slots, acc):
        if slots == 0:
            if left == 0:
                out.append(tuple(acc))
            return
        if i == len(vals):
            return
        v = vals[i]
        lo = vals[-1]
        for c in range(min(slots, left // max(v * v, 1) if v else slots), -1, -1):
            rest = left - c * v * v
            if rest < (slots - c) * lo * lo:
                continue
            if v == 0 and c != slots:
                continue
            walk(i + 1, rest, slots - c, acc + [v] * c)

    walk(0, norm, 24, [])
    return out


def _count_even(key) -> int:
    a_w = {w: len(v) for w, v in _golay_by_weight().items()}
    twos = [v for v in key if v % 4 == 2]
    rest = [v for v in key if v % 4 == 0]
    w = len(twos)
    if w not in a_w:
        return 0
    hist = lambda vs: [vs.count(u) for u in set(vs)]
    nz = sum(1 for v in key if v)
    if w:
        sg = 2 ** (nz - 1)
    else:
        sg = 2 ** nz if sum(key) % 8 == 0 else 0
    return a_w[w] * _perms(hist(twos)) * _perms(hist(rest)) * sg


def _count_odd(key) -> int:
    # every arrangement paired with every codeword gives one candidate; count
    # the candidates whose coordinate sum is 4 mod 8
    a_w = {w: len(v) for w, v in _golay_by_weight().items()}
    distinct = sorted(set(key))
    mult = [key.count(u) for u in distinct]
    total = 0

    def walk(i, take, chosen):
        nonlocal total
        if i == len(distinct):
            if take not in a_w:
                return
            s = 0
            for u, c, k in zip(distinct, mult, chosen):
                on = u if u % 4 == 3 else -u   # on the codeword: x = 3 mod 4
                off = u if u % 4 == 1 else -u  # elsewhere:       x = 1 mod 4
                s += k * on + (c - k) * off
            if s % 8 == 4:
                total += a_w[take] * _perms(chosen) * _perms(
                    [c - k for c, k in zip(mult, chosen)])
            return
        for k in range(mult[i] + 1):
            walk(i + 1, take + k, chosen + [k])

    walk(0, 0, [])
    return total


@lru_cache(maxsize=None)
def shell_classes(m: int) -> tuple:
    """(key, count) for every class of shell m, key = magnitudes sorted desc."""
    out = []
    for parity in (0, 1):
        for key in _multisets(16 * m, parity):
            n = _count_even(key) if parity == 0 else _count_odd(key)
            if n:
                out.append((key, n))
    return tuple(sorted(out))


# --------------------------------------------------------------------------
# uniform Leech points
# --------------------------------------------------------------------------

def _uniform_perm_rows(rng, n: int, width: int) -> np.ndarray:
    return np.argsort(rng.random((n, width)), axis=1)


def sample_class(key, n: int, rng) -> np.ndarray:
    """n uniform lattice points whose |x| multiset is `key` -> int8 [n][24]."""
    key = tuple(int(v) for v in key)
    if n == 0:
        return np.zeros((0, 24), dtype=np.int8)
    if key[0] % 2 == 0:
        twos = np.array([v for v in key if v % 4 == 2], dtype=np.int64)
        fours = np.array([v for v in key if v % 4 == 0], dtype=np.int64)
        w = twos.size
        words = _golay_by_weight()[w]
        pick = words[rng.integers(0, words.size, n)]
        onsupp = ((pick[:, None] >> np.arange(24)) & 1).astype(bool)
        # positions on the support in increasing order, then the rest
        order = np.argsort(~onsupp, axis=1, kind="stable")
        vals = np.empty((n, 24), dtype=np.int64)
        if w:
            vals[:, :w] = twos[_uniform_perm_rows(rng, n, w)]
        if 24 - w:
            vals[:, w:] = fours[_uniform_perm_rows(rng, n, 24 - w)]
        x = np.empty((n, 24), dtype=np.int64)
        np.put_along_axis(x, order, vals, axis=1)
        x *= np.where(rng.random((n, 24)) < 0.5, -1, 1)
        if w:
            bad = np.mod(x.sum(axis=1), 8) != 0
            first = np.argmax(onsupp, axis=1)
            rows = np.nonzero(bad)[0]
            x[rows, first[rows]] *= -1
        return x.astype(np.int8)
    mags = np.array(key, dtype=np.int64)
    out = np.empty((n, 24), dtype=np.int64)
    todo = np.arange(n)
    bits = _golay_bits()
    while todo.size:
        k = todo.size
        a = mags[_uniform_perm_rows(rng, k, 24)]
        c = bits[rng.integers(0, bits.shape[0], k)].astype(np.int64)
        want = 1 + 2 * c  # residue mod 4 of each coordinate
        x = np.where(np.mod(a, 4) == want, a, -a)
        ok = np.mod(x.sum(axis=1), 8) == 4
        out[todo[ok]] = x[ok]
        todo = todo[~ok]
    return out.astype(np.int8)


def sample_shells(shells: np.ndarray, rng) -> np.ndarray:
    """One uniform lattice point per entry of `shells` -> int8 [n][24]."""
    shells = np.asarray(shells).reshape(-1)
    out = np.zeros((shells.size, 24), dtype=np.int8)
    for m in np.unique(shells):
        idx = np.nonzero(shells == m)[0]
        if m == 0:
            continue
        cl = shell_classes(int(m))
        counts = np.array([float(c) for _, c in cl])
        choice = rng.choice(len(cl), size=idx.size, p=counts / counts.sum())
        for ci in np.unique(choice):
            sub = idx[choice == ci]
            out[sub] = sample_class(cl[ci][0], sub.size, rng)
    return out


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def _shells_cfg1(rng, n):
    return rng.integers(2, 4, n)


def _shells_low(rng, n):
    ms = np.arange(2, 7)
    p = 2.0 ** -ms
    return rng.choice(ms, size=n, p=p / p.sum())


def _shells_ball(rng, n):
    ms = np.arange(2, 13)
    p = 2.0 ** -ms
    return rng.choice(ms, size=n, p=p / p.sum())


def leech_matrix(rows: int, cols: int, cfg: int, key=None, zero_rate: float = None) -> dict:
    """Leech workload: coords int8 [R][nb][24], scale fp16 bits [R],
    tail fp16 bits [R][cols % 24].  cfg 1 uses shells {2,3} and 2% origin
    blocks; cfg 3, 4 and 5 use shells 2..6 with P(m) ~ 2^-m; cfg 6 the whole
    ball, shells 2..12 with P(m) ~ 2^-m (about 1 % of blocks on shells >= 9)."""
    base = [0, cfg] if key is None else [0, cfg] + list(key)
    nb, tau = cols // 24, cols % 24
    r_c = rng_for(*base, ARR_COORDS, rows, cols)
    shells = (_shells_cfg1(r_c, rows * nb) if cfg == 1 else
              _shells_ball(r_c, rows * nb) if cfg == 6 else _shells_low(r_c, rows * nb))
    coords = sample_shells(shells, r_c).reshape(rows, nb, 24)
    zr = (0.02 if cfg == 1 else 0.0) if zero_rate is None else zero_rate
    if zr:
        zero = rng_for(*base, ARR_ZERO, rows, cols).random((rows, nb)) < zr
        coords[zero] = 0
    scale = fp16_bits(np.abs(rng_for(*base, ARR_SCALE, rows, cols).standard_normal(rows)) * 0.02)
    tail = fp16_bits(rng_for(*base, ARR_AUX, rows, cols).standard_normal((rows, tau)) * 0.02)
    return {"coords": coords, "scale": scale, "tail": tail, "rows": rows, "cols": cols}


def activations(cols: int, batch: int, cfg: int, key=None, rows: int = 0) -> np.ndarray:
    base = [0, cfg] if key is None else [0, cfg] + list(key)
    r = rng_for(*base, ARR_X, rows, cols)
    return fp16_bits(r.standard_normal((batch, cols)))


def bpdq_matrix(rows: int, cols: int, cfg: int = 2, group: int = 256) -> dict:
    r = rng_for(0, cfg, ARR_AUX, rows, cols)
    codes = r.integers(0, 1 << 32, size=(cols // 16, rows), dtype=np.uint64).astype(np.uint32)
    coeffs = fp16_bits(rng_for(0, cfg, ARR_TABLE, rows, cols).standard_normal(
        (cols // group, 3, rows)) * 0.02)
    return {"codes": codes, "coeffs": coeffs, "rows": rows, "cols": cols}


def dense_matrix(rows: int, cols: int, cfg: int = 2) -> np.ndarray:
    r = rng_for(0, cfg, ARR_DENSE, rows, cols)
    return fp16_bits(r.standard_normal((rows, cols)) * 0.02)


def trellis_matrix(rows: int, cols: int, cfg: int = 4) -> dict:
    r = rng_for(0, cfg, ARR_AUX, rows, cols)
    bits = r.integers(0, 1 << 32, size=(rows, cols // 16), dtype=np.uint64).astype(np.uint32)
    table = fp16_bits(rng_for(0, cfg, ARR_TABLE).standard_normal(1 << 16))
    scale = fp16_bits(np.abs(rng_for(0, cfg, ARR_SCALE, rows, cols).standard_normal(rows)) * 0.02)
    return {"bits": bits, "table": table, "scale": scale, "rows": rows, "cols": cols}


def qwen3_8b_matrix(layer: int, matrix: int) -> dict:
    name, rows, cols = QWEN3_8B_MATRICES[matrix]
    d = leech_matrix(rows, cols, 5, key=(layer, matrix))
    d["name"] = name
    return d


def renorm_bits(v) -> np.ndarray:
    """fp16((v - mean v) / std v) with mean and std in float64: the
    renormalization between the matrices of the stack."""
    v = np.asarray(v, dtype=np.float64)
    return fp16_bits((v - v.mean()) / v.std())
