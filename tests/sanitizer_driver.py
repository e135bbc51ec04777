"""Run the library's host code (the expanders, the class table, the 47-bit
rank) from a build instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer, loaded by ctypes, and check every result against
the oracle's own unpackers.

    python tests/sanitizer_driver.py <path to the instrumented host library>

Run it with the sanitizer runtimes preloaded (tests/test_host_sanitizers.py
does): a heap over-read, a use after free or an undefined operation in the C++
aborts the process with the sanitizer's report.  Prints "SANITIZED OK" at the
end.  Nothing here loads the HIP library or uses a GPU.
"""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import lattice_points  # noqa: E402
import synth  # noqa: E402
from oracle import index as oi  # noqa: E402
from oracle import layout, leech  # noqa: E402

LVQ_OK, LVQ_E_NOT_LEECH, LVQ_E_NORM, LVQ_E_SHAPE = 0, -4, -5, -2


def load(path):
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "lvq_class_table": (i, [vp]),
        "lvq_layout_bytes": (sz, [i, i]),
        "lvq_expand": (i, [vp, vp, vp, i, i, vp]),
        "lvq_expand_gain": (i, [vp, vp, vp, vp, i, i, vp]),
        "lvq_layout_bytes_lp2": (sz, [i, i]),
        "lvq_expand_lp2": (i, [vp, vp, vp, i, i, vp]),
        "lvq_lp2x_exceptions": (i, [vp, i, i, vp]),
        "lvq_layout_bytes_lp2x": (sz, [i, i, sz]),
        "lvq_expand_lp2x": (i, [vp, vp, vp, i, i, sz, vp]),
        "lvq_layout_bytes_direct": (sz, [i, i]),
        "lvq_expand_direct": (i, [vp, vp, vp, i, i, vp]),
        "lvq_layout_bytes_onehot": (sz, [i, i]),
        "lvq_expand_onehot": (i, [vp, vp, vp, i, i, vp]),
        "lvq_rank": (i, [vp, sz, vp]),
        "lvq_last_error_index": (i, [vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


def ptr(a):
    return None if a is None else a.ctypes.data


def whole_ball_matrix(rows, nb, tau, seed, max_shell=12):
    """Blocks of every class up to max_shell (random permutations and signs),
    some origin blocks, fp16 scales and tails."""
    rng = np.random.default_rng(seed)
    cl = leech.classes()
    ids = [c for c in range(1, leech.NUM_CLASSES) if cl[c]["m"] <= max_shell]
    pick = rng.choice(ids, rows * nb)
    pick[rng.random(rows * nb) < 0.05] = 0
    coords = np.zeros((rows * nb, 24), dtype=np.int8)
    for cid in np.unique(pick):
        sel = np.nonzero(pick == cid)[0]
        if cid:
            coords[sel] = synth.sample_class(cl[cid]["key"], sel.size, rng)
    return (coords.reshape(rows, nb, 24), synth.fp16_bits(rng.standard_normal(rows) * 0.02),
            synth.fp16_bits(rng.standard_normal((rows, tau)) * 0.02) if tau else None)


def expand(lib, fn, nbytes, coords, scale, tail, rows, cols):
    blob = np.full(nbytes, 0xA5, dtype=np.uint8)  # every byte must be written
    e = fn(ptr(coords), ptr(scale), ptr(tail), rows, cols, blob.ctypes.data)
    assert e == LVQ_OK, e
    return blob


def check_lp3(lib, coords, scale, tail, rows, cols):
    blob = expand(lib, lib.lvq_expand, lib.lvq_layout_bytes(rows, cols), coords, scale, tail,
                  rows, cols)
    got = layout.unpack_blob(blob, rows, cols)
    assert not got["bad_slot"].any()
    exp = layout.expected_planes(coords.reshape(-1, 24).astype(np.int64))
    for k in ("cls", "sign", "r0", "r1", "r2"):
        assert np.array_equal(np.asarray(got[k]), np.asarray(exp[k])), k
    assert np.array_equal(got["scale"], scale)
    if tail is not None:
        assert np.array_equal(got["tail"], tail)
    assert np.array_equal(got["table"], layout.class_table())
    return blob


def check_layout(lib, kind, coords, scale, tail, rows, cols):
    fn, nb_fn, unpack = {
        "lp2": (lib.lvq_expand_lp2, lib.lvq_layout_bytes_lp2, layout.unpack_lp2),
        "direct": (lib.lvq_expand_direct, lib.lvq_layout_bytes_direct, layout.unpack_direct),
        "onehot": (lib.lvq_expand_onehot, lib.lvq_layout_bytes_onehot, layout.unpack_onehot),
    }[kind]
    blob = expand(lib, fn, nb_fn(rows, cols), coords, scale, tail, rows, cols)
    got = unpack(blob, rows, cols)
    assert np.array_equal(got["coords"], coords), kind


def check_lp2x(lib, coords, scale, tail, rows, cols):
    n = ctypes.c_size_t()
    assert lib.lvq_lp2x_exceptions(ptr(coords), rows, cols, ctypes.byref(n)) == LVQ_OK
    blob = np.full(lib.lvq_layout_bytes_lp2x(rows, cols, n.value), 0xA5, dtype=np.uint8)
    assert lib.lvq_expand_lp2x(ptr(coords), ptr(scale), ptr(tail), rows, cols, n.value,
                               blob.ctypes.data) == LVQ_OK
    got = layout.unpack_lp2x(blob, rows, cols, n.value)
    assert np.array_equal(got["coords"], coords)
    return n.value


def main():
    lib = load(sys.argv[1])
    table = np.zeros(leech.NUM_CLASSES, dtype=np.uint64)
    assert lib.lvq_class_table(table.ctypes.data) == LVQ_OK
    assert np.array_equal(table, layout.class_table())

    # every minimal vector, through LP3, LP2, direct and one-hot, with a tail
    pts = lattice_points.shell2_vectors()
    rows, nb, tau = 910, 216, 5  # 196,560 blocks
    assert rows * nb == pts.shape[0]
    rng = np.random.default_rng(0)
    coords = pts[rng.permutation(pts.shape[0])].reshape(rows, nb, 24)
    scale = synth.fp16_bits(rng.standard_normal(rows))
    tail = synth.fp16_bits(rng.standard_normal((rows, tau)))
    cols = 24 * nb + tau
    check_lp3(lib, coords, scale, tail, rows, cols)
    for kind in ("lp2", "direct", "onehot"):
        check_layout(lib, kind, coords, scale, tail, rows, cols)
    print("shell 2: LP3, LP2, direct, one-hot round trips", flush=True)

    # the whole ball (every class of shells 2..12), ragged shapes and tails
    for seed, (rows, nb, tau) in enumerate([(37, 20, 7), (1, 1, 0), (5, 3, 23), (64, 65, 16),
                                             (3, 0, 9), (0, 4, 1)]):
        coords, scale, tail = whole_ball_matrix(rows, nb, tau, seed)
        cols = 24 * nb + tau
        if rows and nb:
            check_lp3(lib, coords, scale, tail, rows, cols)
            check_lp2x(lib, coords, scale, tail, rows, cols)
            for kind in ("direct", "onehot"):
                check_layout(lib, kind, coords, scale, tail, rows, cols)
            small = whole_ball_matrix(rows, nb, tau, 100 + seed, max_shell=8)
            check_layout(lib, "lp2", *small, rows, cols)
        else:
            for fn, nb_fn in ((lib.lvq_expand, lib.lvq_layout_bytes),
                              (lib.lvq_expand_direct, lib.lvq_layout_bytes_direct)):
                expand(lib, fn, nb_fn(rows, cols), coords, scale, tail, rows, cols)
    print("whole ball: LP3, LP2X, direct, one-hot, LP2 round trips", flush=True)

    # shape-gain: the gain bit rides in bit 15 of the class id
    coords, scale, tail = whole_ball_matrix(9, 11, 4, 7)
    rows, cols = 9, 24 * 11 + 4
    gbits = np.random.default_rng(3).integers(0, 2, (rows, 11)).astype(np.uint8)
    blob = np.full(lib.lvq_layout_bytes(rows, cols), 0xA5, dtype=np.uint8)
    assert lib.lvq_expand_gain(ptr(coords), ptr(gbits), ptr(scale), ptr(tail), rows, cols,
                               blob.ctypes.data) == LVQ_OK
    got = layout.unpack_blob(blob, rows, cols)
    exp = layout.expected_planes(coords.reshape(-1, 24).astype(np.int64))
    assert np.array_equal(np.asarray(got["cls"]) & 0x7FFF, np.asarray(exp["cls"]))
    assert np.array_equal(np.asarray(got["cls"]) >> 15, gbits.reshape(-1))
    print("shape-gain expansion", flush=True)

    # the 47-bit rank against the oracle's
    coords, _, _ = whole_ball_matrix(4, 50, 0, 11)
    out = np.zeros(200, dtype=np.uint64)
    assert lib.lvq_rank(ptr(coords), 200, out.ctypes.data) == LVQ_OK
    for i, x in enumerate(coords.reshape(-1, 24)):
        assert int(out[i]) == oi.rank(x.astype(np.int64)), i
    print("rank", flush=True)

    # refusals: a non-lattice block, a block past shell 12, a class LP2 cannot hold
    coords, scale, tail = whole_ball_matrix(3, 4, 0, 5, max_shell=6)
    bad = coords.copy()
    bad[1, 2] = 0
    bad[1, 2, 0] = 2  # a single 2: not a lattice point
    blob = np.zeros(lib.lvq_layout_bytes(3, 96), dtype=np.uint8)
    assert lib.lvq_expand(ptr(bad), ptr(scale), None, 3, 96, blob.ctypes.data) == LVQ_E_NOT_LEECH
    r, b = ctypes.c_int(), ctypes.c_int()
    lib.lvq_last_error_index(ctypes.byref(r), ctypes.byref(b))
    assert (r.value, b.value) == (1, 2)
    far = coords.copy()
    far[2, 0] = 0
    far[2, 0, :2] = [12, 12]  # shell 18
    assert lib.lvq_expand(ptr(far), ptr(scale), None, 3, 96, blob.ctypes.data) == LVQ_E_NORM
    big, s2, _ = whole_ball_matrix(2, 3, 0, 6)
    big[0, 0] = 0
    big[0, 0, :3] = [12, 4, 4]  # (12, 4, 4, 0..): distinct magnitudes past LP2's reach
    if leech.is_leech(big[0, 0]):
        lp2 = np.zeros(lib.lvq_layout_bytes_lp2(2, 72), dtype=np.uint8)
        assert lib.lvq_expand_lp2(ptr(big), ptr(s2), None, 2, 72, lp2.ctypes.data) != LVQ_OK
    print("refusals", flush=True)
    print("SANITIZED OK", flush=True)


if __name__ == "__main__":
    main()
