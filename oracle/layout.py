"""Expected logical planes of a Leech block, and an independent unpacker of
the packed blob written by the expander (oracle; test infrastructure).

Logical record ("LP3", 112 bits per 24-weight block, the size of the served
record the Tetra summary describes for the earlier kernel, arXiv 2609.35465,
section 2: each code unfolded at load time into a 112-bit record):
  cls    16 bits  class id in the canonical order of oracle.leech.classes()
  sign   24 bits  bit j = [x_j < 0]  (a zero coordinate has sign 0)
  R0..R2 3 x 24   bit j of R_i = bit i of rank_j, where rank_j is the index of
                  |x_j| in the class's ascending list of distinct magnitudes
Decoding: x_j = (1 - 2 sign_j) * mags(cls)[rank_j].  The class is read once
per block, not per weight (arXiv 2609.02652, related-work paragraph on
lookup-table kernels: a Leech class is a permutation pattern, not a value).

Logical class table entry (8 bytes, little-endian u64): bytes 0..4 hold the
ascending distinct magnitudes padded with 0, byte 7 holds m | parity << 7.

Physical blob (the expander's packing; this module re-reads it from the byte
layout alone).  nb = K // 24 blocks per row, tau = K % 24 tail columns; every
section starts at a multiple of 256 bytes:
  table  u64 [302]          the logical class table
  codes  u32 [R][nb][3]     word w of block (r, k) carries coordinates 8w..8w+7
  cls    u16 [R][nb]
  scale  fp16 [R]
  tail   fp16 [R][tau]
Inside code word w, slot n (0..7) is coordinate j = 8w + 2 (n % 4) + n // 4
(slots v and v + 4 carry two adjacent columns):
  bits 4n .. 4n+2          table slot of the coordinate: rank + 1 (1..5)
  bit (4n + 11) mod 32     1 if x_j >= 0, 0 if x_j < 0

The compact LP2 / LP2X layouts, the table-free direct layout and the
one-hot layout (rank-indicator masks) have their own unpackers below
(sections_*, unpack_*), each read from its byte layout alone.  Direct layout: every coordinate of a lattice point has the block's
parity p, so |x_j| = 2 e_j + p with e_j = 0..6 in the ball; a 16-byte record
holds p, e_j and the sign of each coordinate, and no class table is needed.
"""
import numpy as np

from . import leech

ALIGN = 256
TABLE_ENTRIES = leech.NUM_CLASSES


def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def class_table() -> np.ndarray:
    out = np.zeros(TABLE_ENTRIES, dtype=np.uint64)
    for c in leech.classes():
        b = [0] * 8
        for i, m in enumerate(c["mags"]):
            b[i] = m
        b[7] = c["m"] | (c["parity"] << 7)
        out[c["id"]] = np.uint64(int.from_bytes(bytes(b), "little"))
    return out


def expected_planes_loop(blocks) -> dict:
    """blocks int [n][24] (lattice points) -> cls, sign, r0, r1, r2 (each [n]);
    one coordinate at a time, for small inputs."""
    blocks = np.asarray(blocks, dtype=np.int64).reshape(-1, 24)
    n = blocks.shape[0]
    cls = np.zeros(n, dtype=np.int64)
    sign = np.zeros(n, dtype=np.int64)
    r = [np.zeros(n, dtype=np.int64) for _ in range(3)]
    info = leech.classes()
    for i in range(n):
        x = blocks[i]
        cid = leech.class_of(x)
        mags = info[cid]["mags"]
        cls[i] = cid
        for j in range(24):
            if x[j] < 0:
                sign[i] |= 1 << j
            rank = mags.index(abs(int(x[j])))
            for p in range(3):
                if (rank >> p) & 1:
                    r[p][i] |= 1 << j
    return {"cls": cls, "sign": sign, "r0": r[0], "r1": r[1], "r2": r[2]}


def expected_planes(blocks) -> dict:
    """Same result as expected_planes_loop, vectorized per class for large inputs."""
    blocks = np.asarray(blocks, dtype=np.int64).reshape(-1, 24)
    n = blocks.shape[0]
    mag = np.abs(blocks)
    keys = -np.sort(-mag, axis=1)
    uniq, inv = np.unique(keys, axis=0, return_inverse=True)
    index = leech.class_index()
    info = leech.classes()
    cls = np.empty(n, dtype=np.int64)
    rank = np.empty((n, 24), dtype=np.int64)
    inv = inv.reshape(-1)
    for u in range(uniq.shape[0]):
        cid = index[tuple(int(v) for v in uniq[u])]
        sel = inv == u
        cls[sel] = cid
        rank[sel] = np.searchsorted(np.array(info[cid]["mags"]), mag[sel])
    bitw = np.int64(1) << np.arange(24, dtype=np.int64)
    out = {"cls": cls, "sign": ((blocks < 0) * bitw).sum(axis=1)}
    for p in range(3):
        out["r%d" % p] = (((rank >> p) & 1) * bitw).sum(axis=1)
    return out


def decode_planes(planes: dict) -> np.ndarray:
    """Inverse of expected_planes: planes -> int coordinates [n][24]."""
    info = leech.classes()
    n = len(planes["cls"])
    out = np.zeros((n, 24), dtype=np.int64)
    for i in range(n):
        mags = info[int(planes["cls"][i])]["mags"]
        for j in range(24):
            rank = sum(((int(planes["r%d" % p][i]) >> j) & 1) << p for p in range(3))
            v = mags[rank]
            out[i, j] = -v if (int(planes["sign"][i]) >> j) & 1 else v
    return out


def sections(rows: int, cols: int) -> dict:
    nb, tau = cols // 24, cols % 24
    off = {}
    pos = 0
    for name, size in (("table", TABLE_ENTRIES * 8), ("codes", rows * nb * 12),
                       ("cls", rows * nb * 2), ("scale", rows * 2),
                       ("tail", rows * tau * 2)):
        off[name] = pos
        pos += _align(size)
    off["total"] = pos
    return off


def logical_bytes(rows: int, cols: int) -> int:
    """LP3 weight bytes: 14 per block, 2 per row (scale), 2 per tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (14 * nb + 2 + 2 * tau)


def unpack_blob(blob, rows: int, cols: int) -> dict:
    """Parse the physical blob into logical planes, scales, tails and table."""
    buf = np.frombuffer(bytes(blob), dtype=np.uint8)
    off = sections(rows, cols)
    assert buf.size == off["total"], (buf.size, off["total"])
    nb, tau = cols // 24, cols % 24
    table = buf[off["table"]: off["table"] + TABLE_ENTRIES * 8].view("<u8").copy()
    words = buf[off["codes"]: off["codes"] + rows * nb * 12].view("<u4").reshape(rows * nb, 3)
    cls = buf[off["cls"]: off["cls"] + rows * nb * 2].view("<u2").astype(np.int64)
    scale = buf[off["scale"]: off["scale"] + rows * 2].view("<u2").copy()
    tail = buf[off["tail"]: off["tail"] + rows * tau * 2].view("<u2").reshape(rows, tau).copy()
    n = rows * nb
    sign = np.zeros(n, dtype=np.int64)
    rp = [np.zeros(n, dtype=np.int64) for _ in range(3)]
    bad = np.zeros(n, dtype=bool)
    for w in range(3):
        word = words[:, w].astype(np.int64)
        for slot in range(8):
            j = 8 * w + 2 * (slot % 4) + slot // 4
            t = (word >> (4 * slot)) & 7
            nonneg = (word >> ((4 * slot + 11) % 32)) & 1
            rank = t - 1
            bad |= (t == 0) | (t > 5)
            sign |= (1 - nonneg) << j
            for p in range(3):
                rp[p] |= ((rank >> p) & 1) << j
    return {"table": table, "cls": cls, "sign": sign, "r0": rp[0], "r1": rp[1],
            "r2": rp[2], "scale": scale, "tail": tail, "bad_slot": bad}


# --------------------------------------------------------------------------
# LP2: two rank planes, the class inside the code record
# --------------------------------------------------------------------------
#
# Physical LP2 blob (the expander's packing for blocks whose class has at most
# four distinct magnitudes and an id below 256, which covers shells m <= 8).
# The paper reports smaller in-VRAM layouts than its served record (section 1,
# contribution C2: layouts of 5.51, 4.80, 4.34 and 3.59 bits per weight); the
# bit layout below is this library's:
#   table  u64 [302]        as LP3
#   codes  u32 [R][nb][3]   12 bytes per block, no class section
#   scale  fp16 [R], tail fp16 [R][tau]
# In word w, coordinate j = 8w + 2v + h (v = 0..3, h = 0, 1):
#   bits 2v+16h .. 2v+16h+1   rank (0..3)
#   bit 8+2v+16h              1 if x_j >= 0
# Word 0, odd bits: class id bit 2i at bit 9+2i, bit 2i+1 at bit 25+2i (i<4).

def sections_lp2(rows: int, cols: int) -> dict:
    nb, tau = cols // 24, cols % 24
    off = {}
    pos = 0
    for name, size in (("table", TABLE_ENTRIES * 8), ("codes", rows * nb * 12),
                       ("scale", rows * 2), ("tail", rows * tau * 2)):
        off[name] = pos
        pos += _align(size)
    off["total"] = pos
    return off


def lp2_bytes(rows: int, cols: int) -> int:
    """LP2 weight bytes: 12 per block, 2 per row, 2 per tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (12 * nb + 2 + 2 * tau)


def unpack_lp2(blob, rows: int, cols: int) -> dict:
    """Coordinates int8 [R][nb][24], class ids, scales and tails from an LP2
    blob, read from the byte layout and the oracle's class table alone."""
    buf = np.frombuffer(bytes(blob), dtype=np.uint8)
    off = sections_lp2(rows, cols)
    assert buf.size == off["total"], (buf.size, off["total"])
    nb, tau = cols // 24, cols % 24
    words = buf[off["codes"]: off["codes"] + rows * nb * 12].view("<u4").reshape(rows * nb, 3)
    words = words.astype(np.int64)
    cls = np.zeros(rows * nb, dtype=np.int64)
    for i in range(4):
        cls |= ((words[:, 0] >> (9 + 2 * i)) & 1) << (2 * i)
        cls |= ((words[:, 0] >> (25 + 2 * i)) & 1) << (2 * i + 1)
    classes = leech.classes()
    mags = np.zeros((len(classes), 4), dtype=np.int64)
    for cid, c in enumerate(classes):
        dm = sorted(set(c["key"]))
        mags[cid, : len(dm)] = dm[:4]
    coords = np.zeros((rows * nb, 24), dtype=np.int64)
    for j in range(24):
        w, jj = divmod(j, 8)
        v, h = jj // 2, jj % 2
        rank = (words[:, w] >> (2 * v + 16 * h)) & 3
        nonneg = (words[:, w] >> (8 + 2 * v + 16 * h)) & 1
        mag = mags[cls, rank]
        coords[:, j] = np.where(nonneg == 1, mag, -mag)
    return {"coords": coords.astype(np.int8).reshape(rows, nb, 24), "cls": cls.reshape(rows, nb),
            "scale": buf[off["scale"]: off["scale"] + rows * 2].view("<u2").copy(),
            "tail": buf[off["tail"]: off["tail"] + rows * tau * 2].view("<u2").reshape(rows, tau).copy()}


# --------------------------------------------------------------------------
# LP2X: LP2 plus an exception side channel
# --------------------------------------------------------------------------
#
# After the LP2 sections: exc_off u32 [R + 1] (first entry of each row) and
# 16-byte entries {block index | class id << 16, the block's three code words
# in the LP3 packing above}.  Blocks in the side channel have a zero LP2
# record.

def sections_lp2x(rows: int, cols: int, n_exc: int) -> dict:
    off = sections_lp2(rows, cols)
    off["exc_off"] = off["total"]
    off["exc"] = off["exc_off"] + _align((rows + 1) * 4)
    off["total"] = off["exc"] + _align(n_exc * 16)
    return off


def unpack_lp2x(blob, rows: int, cols: int, n_exc: int) -> dict:
    """Coordinates of an LP2X blob: the LP2 records, then every side-channel
    entry decoded with the LP3 slot layout and the oracle's class table."""
    buf = np.frombuffer(bytes(blob), dtype=np.uint8)
    off = sections_lp2x(rows, cols, n_exc)
    assert buf.size == off["total"], (buf.size, off["total"])
    nb = cols // 24
    head = unpack_lp2(buf[: sections_lp2(rows, cols)["total"]].tobytes(), rows, cols)
    coords = head["coords"].astype(np.int64).reshape(rows * nb, 24) if nb else \
        np.zeros((0, 24), dtype=np.int64)
    exc_off = buf[off["exc_off"]: off["exc_off"] + (rows + 1) * 4].view("<u4")
    ent = buf[off["exc"]: off["exc"] + n_exc * 16].view("<u4").reshape(n_exc, 4)
    classes = leech.classes()
    for r in range(rows):
        for e in range(int(exc_off[r]), int(exc_off[r + 1])):
            k, cid = int(ent[e, 0] & 0xFFFF), int(ent[e, 0] >> 16)
            mags = sorted(set(classes[cid]["key"]))
            x = np.zeros(24, dtype=np.int64)
            for w in range(3):
                word = int(ent[e, 1 + w])
                for slot in range(8):
                    j = 8 * w + 2 * (slot % 4) + slot // 4
                    rank = ((word >> (4 * slot)) & 7) - 1
                    nonneg = (word >> ((4 * slot + 11) % 32)) & 1
                    x[j] = mags[rank] if nonneg else -mags[rank]
            assert not np.any(coords[r * nb + k]), "side-channel block with a main record"
            coords[r * nb + k] = x
    return {"coords": coords.astype(np.int8).reshape(rows, nb, 24), "exc_off": exc_off.copy()}


def sections_direct(rows: int, cols: int) -> dict:
    nb, tau = cols // 24, cols % 24
    off = {}
    pos = 0
    for name, size in (("codes", rows * nb * 16), ("scale", rows * 2), ("tail", rows * tau * 2)):
        off[name] = pos
        pos += _align(size)
    off["total"] = pos
    return off


def direct_bytes(rows: int, cols: int) -> int:
    """Direct-layout weight bytes: 16 per block, 2 per row, 2 per tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (16 * nb + 2 + 2 * tau)


def unpack_direct(blob, rows: int, cols: int) -> dict:
    """Coordinates int8 [R][nb][24], scales and tails from a direct-layout
    blob: no class table.  Each block is four little-endian 32-bit words; the
    block parity p is bit 0 of word 0; coordinate j sits in word (j // 2) // 3
    with view v = (j // 2) % 3 and half h = j % 2, its three magnitude bits
    e at (1 + f + 16 h + 5 v) mod 32 and its sign at (15 + 16 h + 5 v) mod 32,
    and |x_j| = 2 e + p."""
    buf = np.frombuffer(bytes(blob), dtype=np.uint8)
    off = sections_direct(rows, cols)
    assert buf.size == off["total"], (buf.size, off["total"])
    nb, tau = cols // 24, cols % 24
    words = buf[off["codes"]: off["codes"] + rows * nb * 16].view("<u4").reshape(rows * nb, 4)
    words = words.astype(np.int64)
    p = words[:, 0] & 1
    coords = np.zeros((rows * nb, 24), dtype=np.int64)
    for j in range(24):
        pair, h = divmod(j, 2)
        w, v = divmod(pair, 3)
        e = np.zeros(rows * nb, dtype=np.int64)
        for f in range(3):
            e |= ((words[:, w] >> ((1 + f + 16 * h + 5 * v) % 32)) & 1) << f
        neg = (words[:, w] >> ((15 + 16 * h + 5 * v) % 32)) & 1
        mag = 2 * e + p
        coords[:, j] = np.where(neg == 1, -mag, mag)
    return {"coords": coords.astype(np.int8).reshape(rows, nb, 24),
            "words": words.astype(np.uint32).reshape(rows, nb, 4),
            "scale": buf[off["scale"]: off["scale"] + rows * 2].view("<u2").copy(),
            "tail": buf[off["tail"]: off["tail"] + rows * tau * 2].view("<u2").reshape(rows, tau).copy()}


def sections_onehot(rows: int, cols: int) -> dict:
    nb, tau = cols // 24, cols % 24
    off = {}
    pos = 0
    for name, size in (("table", TABLE_ENTRIES * 8), ("codes", rows * nb * 16),
                       ("cls", rows * nb * 2), ("scale", rows * 2), ("tail", rows * tau * 2)):
        off[name] = pos
        pos += _align(size)
    off["total"] = pos
    return off


def onehot_bytes(rows: int, cols: int) -> int:
    """One-hot weight bytes: 16 per block record, 2 per class id, 2 per row,
    2 per tail column."""
    nb, tau = cols // 24, cols % 24
    return rows * (18 * nb + 2 + 2 * tau)


def unpack_onehot(blob, rows: int, cols: int) -> dict:
    """Coordinates int8 [R][nb][24], class ids, scales and tails from a
    one-hot blob, read from the byte layout and the oracle's class table.
    Word i of a block marks the coordinates of rank i + 1 (coordinate 2P at
    bit P, 2P + 1 at bit 16 + P); a coordinate with no mark has rank 0; the
    signs of pairs 3i .. 3i + 2 sit at bits 12 + P - 3i and 28 + P - 3i of
    word i.  A coordinate marked twice is an error (the masks are one-hot)."""
    buf = np.frombuffer(bytes(blob), dtype=np.uint8)
    off = sections_onehot(rows, cols)
    assert buf.size == off["total"], (buf.size, off["total"])
    nb, tau = cols // 24, cols % 24
    n = rows * nb
    words = buf[off["codes"]: off["codes"] + n * 16].view("<u4").reshape(n, 4).astype(np.int64)
    cls = buf[off["cls"]: off["cls"] + n * 2].view("<u2").astype(np.int64)
    classes = leech.classes()
    mags = np.zeros((len(classes), 5), dtype=np.int64)
    for cid, c in enumerate(classes):
        dm = sorted(set(c["key"]))
        mags[cid, : len(dm)] = dm
    coords = np.zeros((n, 24), dtype=np.int64)
    for j in range(24):
        pair, h = divmod(j, 2)
        rank = np.zeros(n, dtype=np.int64)
        marks = np.zeros(n, dtype=np.int64)
        for i in range(4):
            bit = (words[:, i] >> (pair + 16 * h)) & 1
            rank += bit * (i + 1)
            marks += bit
        assert np.all(marks <= 1), "a coordinate marked by two rank masks"
        sw = pair // 3
        neg = (words[:, sw] >> (12 + pair - 3 * sw + 16 * h)) & 1
        mag = mags[cls, rank]
        coords[:, j] = np.where(neg == 1, -mag, mag)
    return {"coords": coords.astype(np.int8).reshape(rows, nb, 24), "cls": cls.reshape(rows, nb),
            "words": words.astype(np.uint32).reshape(rows, nb, 4),
            "table": buf[off["table"]: off["table"] + TABLE_ENTRIES * 8].view("<u8").copy(),
            "scale": buf[off["scale"]: off["scale"] + rows * 2].view("<u2").copy(),
            "tail": buf[off["tail"]: off["tail"] + rows * tau * 2].view("<u2").reshape(rows, tau).copy()}
