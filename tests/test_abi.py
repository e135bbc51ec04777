"""The C ABI on the CPU: exports, the host expander against the oracle, and
argument validation of the device entry points (which return before any HIP
call, so no GPU is needed)."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import dequant_gemv_lvq_amd as lvq
import lattice_points
import synth
from oracle import golay, layout, leech

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "lvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z0-9_]+)\s*\(", text)) - {"if", "sizeof"})


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert set(declared) == set(lvq.EXPORTED)
    for name in declared:
        assert hasattr(lvq.library(), name), name


def test_strerror():
    for code in range(-7, 1):
        assert lvq.strerror(code) and lvq.strerror(code) != "unknown status"
    assert lvq.strerror(-99) == "unknown status"


def test_class_table_matches_oracle():
    assert np.array_equal(lvq.class_table(), layout.class_table())


def test_layout_bytes_matches_oracle():
    for r, c in [(0, 0), (1, 1), (3, 50), (4096, 12288), (4096, 4096), (12288, 4096), (7, 23)]:
        assert lvq.layout_bytes(r, c) == layout.sections(r, c)["total"]
    assert lvq.layout_bytes(-1, 5) == 0 and lvq.layout_bytes(5, -1) == 0


def _check_blob(coords, scale, tail, rows, cols):
    blob = lvq.expand(coords, scale, tail, rows, cols)
    u = layout.unpack_blob(blob, rows, cols)
    exp = layout.expected_planes(np.asarray(coords).reshape(-1, 24))
    assert not u["bad_slot"].any()
    for k in ("cls", "sign", "r0", "r1", "r2"):
        assert np.array_equal(u[k], exp[k]), k
    assert np.array_equal(u["table"], layout.class_table())
    assert np.array_equal(u["scale"], scale)
    if cols % 24:
        assert np.array_equal(u["tail"], tail)
    return blob, u


def test_expand_exhaustive_shell2():
    x = lattice_points.shell2_vectors()
    assert x.shape[0] == 196560
    rows = 196560 // 24
    coords = x.reshape(rows, 24, 24)
    scale = synth.fp16_bits(np.linspace(0.01, 0.03, rows))
    blob, u = _check_blob(coords, scale, None, rows, 576)
    assert np.array_equal(layout.decode_planes(u)[:5000], x[:5000].astype(np.int64))


def test_expand_every_class_with_tail():
    rng = np.random.default_rng(8)
    blocks = [np.zeros((1, 24), dtype=np.int8)]
    for c in leech.classes()[1:]:
        blocks.append(synth.sample_class(c["key"], 3, rng))
    blocks = np.concatenate(blocks)  # 904 blocks
    rows, nb = 8, blocks.shape[0] // 8
    cols = 24 * nb + 13
    coords = blocks[: rows * nb].reshape(rows, nb, 24)
    scale = synth.fp16_bits(rng.random(rows))
    tail = synth.fp16_bits(rng.standard_normal((rows, 13)))
    _check_blob(coords, scale, tail, rows, cols)


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2 ** 31 - 1), rows=st.integers(1, 5), nb=st.integers(0, 9),
       tau=st.integers(0, 23), shells=st.sampled_from([(2, 3), (2, 6), (7, 12)]))
def test_expand_roundtrip_property(seed, rows, nb, tau, shells):
    rng = np.random.default_rng(seed)
    m = rng.integers(shells[0], shells[1] + 1, rows * nb)
    coords = synth.sample_shells(m, rng).reshape(rows, nb, 24)
    zero = rng.random((rows, nb)) < 0.1
    coords[zero] = 0
    scale = synth.fp16_bits(rng.standard_normal(rows))
    tail = synth.fp16_bits(rng.standard_normal((rows, tau)))
    _check_blob(coords, scale, tail, rows, 24 * nb + tau)


def test_expand_errors():
    d = synth.leech_matrix(3, 72, 3, key=(1,))
    c = d["coords"].copy()
    c[1, 2, 0] = -c[1, 2, 0] if c[1, 2, 0] else 2  # breaks the sum or the parity
    if leech.is_leech(c[1, 2]):
        c[1, 2, 5] += 2
    with pytest.raises(lvq.LvqError) as e:
        lvq.expand(c, d["scale"], None, 3, 72)
    assert e.value.code == lvq.LVQ_E_NOT_LEECH and e.value.index == (1, 2)
    far = d["coords"].copy()
    far[2, 0] = 0
    far[2, 0, :2] = [12, 12]  # 3 x (4, 4, 0...) is a lattice point of shell 18
    assert leech.is_leech(far[2, 0])
    with pytest.raises(lvq.LvqError) as e:
        lvq.expand(far, d["scale"], None, 3, 72)
    assert e.value.code == lvq.LVQ_E_NORM and e.value.index == (2, 0)
    blob = lvq.expand(d["coords"], d["scale"], None, 3, 72)
    assert blob.size == lvq.layout_bytes(3, 72)
    assert lvq.last_error_index() == (-1, -1)
    lib = lvq.library()
    buf = np.zeros(lvq.layout_bytes(3, 74), dtype=np.uint8)
    assert lib.lvq_expand(d["coords"].ctypes.data, d["scale"].ctypes.data, None, 3, 74,
                          buf.ctypes.data) == lvq.LVQ_E_NULL  # tail required
    assert lib.lvq_expand(None, d["scale"].ctypes.data, None, 3, 72, buf.ctypes.data) == lvq.LVQ_E_NULL
    assert lib.lvq_expand(None, None, None, -1, 72, buf.ctypes.data) == lvq.LVQ_E_SHAPE
    assert lib.lvq_class_table(None) == lvq.LVQ_E_NULL


def test_device_entry_points_validate_before_launch():
    lib = lvq.library()
    A = 1 << 20  # a fake, 16-byte aligned address; never dereferenced
    assert lib.lvq_gemv(A, 4, 48, A, A, 0, None) == lvq.LVQ_E_BATCH
    assert lib.lvq_gemv(A, 4, 48, A, A, 5, None) == lvq.LVQ_E_BATCH
    assert lib.lvq_gemv(None, 4, 48, A, A, 1, None) == lvq.LVQ_E_NULL
    assert lib.lvq_gemv(A + 4, 4, 48, A, A, 1, None) == lvq.LVQ_E_ALIGN
    assert lib.lvq_gemv(A, -1, 48, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert lib.lvq_gemv(A, 4, 70000, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert lib.lvq_gemv(A, 4, 65537, A, A, 1, None) == lvq.LVQ_E_SHAPE  # batch x cols > 65,536
    assert lib.lvq_gemv(A, 4, 16385, A, A, 4, None) == lvq.LVQ_E_SHAPE
    assert lib.lvq_gemv(A, 0, 48, A, A, 1, None) == lvq.LVQ_OK  # nothing to do
    assert lib.lvq_decode(A, 4, 48, None, None) == lvq.LVQ_E_NULL
    assert lib.lvq_decode(A, 4, 48, A + 8, None) == lvq.LVQ_E_ALIGN
    assert lib.bpdq_gemv(A, A, 16, 100, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert lib.bpdq_gemv(A, A, 16, 256, A, A, 9, None) == lvq.LVQ_E_BATCH
    assert lib.bpdq_gemv(A, None, 16, 256, A, A, 1, None) == lvq.LVQ_E_NULL
    assert lib.bpdq_gemv(A, A, 16, 65536 + 256, A, A, 1, None) == lvq.LVQ_E_SHAPE  # batch x cols
    assert lib.bpdq_gemv(A, A, 16, 16384 + 256, A, A, 4, None) == lvq.LVQ_E_SHAPE
    assert lib.bpdq_gemv(A, A, 1 << 20, 16384, A, A, 1, None) == lvq.LVQ_E_SHAPE  # codes > 2 GiB
    assert lib.trellis_gemv(A, A, A, 16, 300, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert lib.trellis_gemv(A, A, A, 16, 4096, A, A, 4, None) == lvq.LVQ_E_SHAPE
    assert lib.trellis_gemv(A, A, A + 2, 16, 256, A, A, 1, None) == lvq.LVQ_E_ALIGN
    assert lib.fp16_gemv(A, 16, 100, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert lib.fp16_gemv(A, 16, 128, A, None, 1, None) == lvq.LVQ_E_NULL
    assert lib.lvq_stream_read(None, 64, A, None) == lvq.LVQ_E_NULL
    assert lib.lvq_stream_read(A, 64, None, None) == lvq.LVQ_E_NULL
    assert lib.lvq_stream_read(A + 4, 64, A, None) == lvq.LVQ_E_ALIGN
    assert lib.lvq_stream_read(A, 66, A, None) == lvq.LVQ_E_ALIGN
    assert lib.lvq_stream_read_geom(None, 64, A, 256, 1, 1, 1, None) == lvq.LVQ_E_NULL
    assert lib.lvq_stream_read_geom(A + 4, 64, A, 256, 1, 1, 1, None) == lvq.LVQ_E_ALIGN
    assert lib.lvq_stream_read_geom(A, 64, A, 128, 1, 1, 1, None) == lvq.LVQ_E_SHAPE
    assert lib.lvq_stream_read_geom(A, 64, A, 256, 9, 1, 1, None) == lvq.LVQ_E_SHAPE
    assert lib.lvq_stream_read_geom(A, 64, A, 256, 1, 3, 1, None) == lvq.LVQ_E_SHAPE
    # one trip per thread over 2^31 bytes at 256 x 1 loads needs 524,288
    # workgroups, more than the sink holds: refused before any launch
    assert lib.lvq_stream_read_geom(A, 1 << 31, A, 256, 0, 1, 1, None) == lvq.LVQ_E_SHAPE


@pytest.mark.parametrize("name", ["expand", "expand_lp2", "expand_lp2x", "expand_direct",
                                  "expand_onehot", "expand_gain"])
def test_expanders_reject_short_host_arrays(name):
    """Every host expander checks the sizes of coords, scale and tail before
    the native call, so a short array is refused instead of read past."""
    rows, cols = 3, 74  # two blocks and a tail of 2 per row
    d = synth.leech_matrix(rows, cols, 3, key=(5,))
    fn = getattr(lvq, name)

    def call(coords, scale, tail):
        if name == "expand_gain":
            return fn(coords, np.zeros((rows, cols // 24), np.uint8), scale, tail, rows, cols)
        return fn(coords, scale, tail, rows, cols)

    call(d["coords"], d["scale"], d["tail"])  # the full arrays are accepted
    bad = [(d["coords"][:2], d["scale"], d["tail"]),
           (d["coords"], d["scale"][:2], d["tail"]),
           (d["coords"], d["scale"], d["tail"][:2]),
           (d["coords"], d["scale"], None)]
    for coords, scale, tail in bad:
        with pytest.raises(lvq.LvqError) as e:
            call(coords, scale, tail)
        assert e.value.code == lvq.LVQ_E_SHAPE
    if name == "expand_gain":
        with pytest.raises(lvq.LvqError):
            fn(d["coords"], np.zeros(rows, np.uint8), d["scale"], d["tail"], rows, cols)


def test_fused_and_noweights_validate_before_launch():
    import ctypes
    lib = lvq.library()
    A = 1 << 20

    def arr(t, vals):
        return (t * len(vals))(*vals)

    vp, ci = ctypes.c_void_p, ctypes.c_int
    blobs, ys = arr(vp, [A, A, A]), arr(vp, [A, A, A])
    rows = arr(ci, [4, 8, 12])
    f = lib.lvq_gemv_fused
    assert f(0, blobs, rows, 48, A, ys, 1, None) == lvq.LVQ_E_SHAPE
    assert f(lvq.MAX_FUSED + 1, arr(vp, [A] * 5), arr(ci, [4] * 5), 48, A, arr(vp, [A] * 5), 1,
             None) == lvq.LVQ_E_SHAPE
    assert f(3, None, rows, 48, A, ys, 1, None) == lvq.LVQ_E_NULL
    assert f(3, blobs, None, 48, A, ys, 1, None) == lvq.LVQ_E_NULL
    assert f(3, blobs, rows, 48, A, None, 1, None) == lvq.LVQ_E_NULL
    assert f(3, arr(vp, [A, None, A]), rows, 48, A, ys, 1, None) == lvq.LVQ_E_NULL
    assert f(3, blobs, rows, 48, A, arr(vp, [A, A, None]), 1, None) == lvq.LVQ_E_NULL
    assert f(3, blobs, rows, 48, None, ys, 1, None) == lvq.LVQ_E_NULL
    assert f(3, arr(vp, [A, A + 8, A]), rows, 48, A, ys, 1, None) == lvq.LVQ_E_ALIGN
    assert f(3, blobs, rows, 48, A, arr(vp, [A + 4, A, A]), 1, None) == lvq.LVQ_E_ALIGN
    assert f(3, blobs, rows, 48, A + 2, ys, 1, None) == lvq.LVQ_E_ALIGN
    assert f(3, blobs, arr(ci, [4, -1, 12]), 48, A, ys, 1, None) == lvq.LVQ_E_SHAPE
    assert f(3, blobs, rows, -24, A, ys, 1, None) == lvq.LVQ_E_SHAPE
    assert f(3, blobs, rows, 70000, A, ys, 1, None) == lvq.LVQ_E_SHAPE
    assert f(3, blobs, rows, 48, A, ys, 0, None) == lvq.LVQ_E_BATCH
    assert f(3, blobs, rows, 48, A, ys, 5, None) == lvq.LVQ_E_BATCH
    # more rows in the set than an int indexes
    assert f(2, blobs, arr(ci, [1 << 30, 1 << 30]), 48, A, ys, 1, None) == lvq.LVQ_E_SHAPE
    assert f(3, blobs, arr(ci, [0, 0, 0]), 48, A, ys, 1, None) == lvq.LVQ_OK  # nothing to do
    with pytest.raises(ValueError):
        lvq.gemv_fused([A, A], [4], 48, A, [A, A])
    with pytest.raises(lvq.LvqError):
        lvq.gemv_fused([], [], 48, A, [])

    g = lib.lvq_gemv_noweights
    assert g(A, 4, 48, A, A, 0, None) == lvq.LVQ_E_BATCH
    assert g(None, 4, 48, A, A, 1, None) == lvq.LVQ_E_NULL
    assert g(A, 4, 48, A, None, 1, None) == lvq.LVQ_E_NULL
    assert g(A + 4, 4, 48, A, A, 1, None) == lvq.LVQ_E_ALIGN
    assert g(A, -1, 48, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert g(A, 4, 70000, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert g(A, 0, 48, A, A, 1, None) == lvq.LVQ_OK


def test_rotate_validates_before_launch():
    lib = lvq.library()
    A = 1 << 20
    r = lib.lvq_rotate
    assert r(A, None, None, 4096, 1, A, 0, None) == lvq.LVQ_E_BATCH
    assert r(A, None, None, -8, 1, A, 1, None) == lvq.LVQ_E_SHAPE
    assert r(A, None, None, 4096, 0, A, 1, None) == lvq.LVQ_E_SHAPE
    assert r(A, None, None, 33 * 64, 33, A, 1, None) == lvq.LVQ_E_SHAPE   # m > 32
    assert r(A, None, None, 100, 3, A, 1, None) == lvq.LVQ_E_SHAPE       # n % m
    assert r(A, None, None, 3 * 12, 3, A, 1, None) == lvq.LVQ_E_SHAPE    # K = 12
    assert r(None, None, None, 4096, 1, A, 1, None) == lvq.LVQ_E_NULL
    assert r(A, None, None, 4096, 1, None, 1, None) == lvq.LVQ_E_NULL
    assert r(A + 2, None, None, 4096, 1, A, 1, None) == lvq.LVQ_E_ALIGN
    assert r(A, A + 4, None, 4096, 1, A, 1, None) == lvq.LVQ_E_ALIGN
    assert r(A, None, A + 8, 3 * 1024, 3, A, 1, None) == lvq.LVQ_E_ALIGN
    assert r(A, None, None, 0, 1, A, 1, None) == lvq.LVQ_OK              # nothing to do
    # m > 1: y must not overlap x (the m workgroups of a row all read x)
    assert r(A, None, None, 3 * 1024, 3, A, 1, None) == lvq.LVQ_E_SHAPE


def test_rank_matches_the_oracle():
    from oracle import index as oi
    rng = np.random.default_rng(48)
    idx = [0, 1, oi.total() - 1, int(oi.block_offsets()[4096])]
    idx += [int(v) for v in rng.integers(0, oi.total(), 400)]
    pts = np.stack([oi.unrank(i) for i in idx])
    got = lvq.rank(pts)
    assert [int(v) for v in got] == idx
    # shell-2 points from the classical construction: distinct ranks, and a
    # sample agrees with the oracle's rank
    pts2 = np.stack([synth.sample_class(c["key"], 300, rng)
                     for c in leech.classes() if c["m"] == 2]).reshape(-1, 24)
    r2 = lvq.rank(pts2)
    for p, r in list(zip(pts2, r2))[::37]:
        assert int(r) == oi.rank(p)
    with pytest.raises(lvq.LvqError):
        bad = pts[:1].copy()
        bad[0, 0] += 2  # breaks the sum rule
        lvq.rank(bad)
    far = np.zeros((1, 24), dtype=np.int8)
    far[0, :2] = [12, 12]  # a lattice point beyond shell 12... if it is one
    if leech.is_leech(far[0]):
        with pytest.raises(lvq.LvqError):
            lvq.rank(far)


def test_expand_gain_stores_the_gain_bit():
    rows, nb, tau = 5, 7, 3
    d = synth.leech_matrix(rows, 24 * nb + tau, 3)
    g = np.random.default_rng(1).integers(0, 2, (rows, nb)).astype(np.uint8)
    blob = lvq.expand_gain(d["coords"], g, d["scale"], d["tail"], rows, 24 * nb + tau)
    plain = lvq.expand(d["coords"], d["scale"], d["tail"], rows, 24 * nb + tau)
    sec = layout.sections(rows, 24 * nb + tau)
    cls_g = blob[sec["cls"]: sec["cls"] + rows * nb * 2].view(np.uint16)
    cls_p = plain[sec["cls"]: sec["cls"] + rows * nb * 2].view(np.uint16)
    assert np.array_equal(cls_g & 0x7FFF, cls_p)
    assert np.array_equal(cls_g >> 15, g.reshape(-1))
    # everything else is the same blob
    mask = np.ones(blob.size, dtype=bool)
    mask[sec["cls"]: sec["cls"] + rows * nb * 2] = False
    assert np.array_equal(blob[mask], plain[mask])
    g[1, 2] = 2
    with pytest.raises(lvq.LvqError):
        lvq.expand_gain(d["coords"], g, d["scale"], d["tail"], rows, 24 * nb + tau)


def test_unfold_and_gain_gemv_validate_before_launch():
    lib = lvq.library()
    A = 1 << 20
    assert lib.lvq_unfold(None, 4, A, A, None) == lvq.LVQ_E_NULL
    assert lib.lvq_unfold(A, 4, None, A, None) == lvq.LVQ_E_NULL
    assert lib.lvq_unfold(A + 8, 4, A, A, None) == lvq.LVQ_E_ALIGN
    assert lib.lvq_unfold(A, 0, A, A, None) == lvq.LVQ_OK
    g = lib.lvq_gemv_gain
    assert g(A, 4, 48, 1.0, 2.0, A, A, 0, None) == lvq.LVQ_E_BATCH
    assert g(None, 4, 48, 1.0, 2.0, A, A, 1, None) == lvq.LVQ_E_NULL
    assert g(A + 4, 4, 48, 1.0, 2.0, A, A, 1, None) == lvq.LVQ_E_ALIGN
    assert g(A, 0, 48, 1.0, 2.0, A, A, 1, None) == lvq.LVQ_OK
    assert lib.lvq_rank(None, 3, A) == lvq.LVQ_E_NULL


@pytest.mark.parametrize("rows,nb,tau,cfg", [(7, 11, 5, 3), (33, 170, 0, 4), (4, 3, 23, 1)])
def test_expand_lp2_round_trips_through_the_oracle_unpacker(rows, nb, tau, cfg):
    cols = 24 * nb + tau
    d = synth.leech_matrix(rows, cols, cfg, key=(rows, nb, tau))
    blob = lvq.expand_lp2(d["coords"], d["scale"], d["tail"], rows, cols)
    assert blob.size == lvq.layout_bytes_lp2(rows, cols) == layout.sections_lp2(rows, cols)["total"]
    u = layout.unpack_lp2(blob, rows, cols)
    assert np.array_equal(u["coords"], d["coords"])
    assert np.array_equal(u["scale"], d["scale"]) and np.array_equal(u["tail"], d["tail"])
    assert np.array_equal(u["cls"], np.vectorize(lambda i: i)(
        [[leech.class_of(b) for b in row] for row in d["coords"]]))


def test_expand_lp2_every_small_class_and_the_refusals():
    rng = np.random.default_rng(9)
    ok = [c for c in leech.classes() if c["id"] < 256 and len(set(c["key"])) <= 4]
    pts = np.stack([synth.sample_class(c["key"], 1, rng)[0] if c["id"] else np.zeros(24, np.int8)
                    for c in ok])
    rows = len(ok)
    scale = synth.fp16_bits(np.ones(rows))
    blob = lvq.expand_lp2(pts.reshape(rows, 1, 24), scale, None, rows, 24)
    assert np.array_equal(layout.unpack_lp2(blob, rows, 24)["coords"].reshape(rows, 24), pts)
    # a class with five distinct magnitudes is refused, and reported
    five = next(c for c in leech.classes() if len(set(c["key"])) == 5)
    x = np.zeros((2, 2, 24), dtype=np.int8)
    x[1, 1] = synth.sample_class(five["key"], 1, rng)[0]
    with pytest.raises(lvq.LvqError) as e:
        lvq.expand_lp2(x, synth.fp16_bits(np.ones(2)), None, 2, 48)
    assert e.value.code == lvq.LVQ_E_LAYOUT and e.value.index == (1, 1)
    assert lvq.strerror(lvq.LVQ_E_LAYOUT).startswith("a block's class")


def _all_class_coords(rows, nb, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, leech.NUM_CLASSES, rows * nb)
    cl = leech.classes()
    coords = np.zeros((rows * nb, 24), dtype=np.int8)
    for cid in np.unique(ids):
        sel = np.nonzero(ids == cid)[0]
        if cid:
            coords[sel] = synth.sample_class(cl[cid]["key"], sel.size, rng)
    return coords.reshape(rows, nb, 24), ids


@pytest.mark.parametrize("src", ["ball", "all_classes"])
def test_expand_lp2x_round_trips_through_the_oracle_unpacker(src):
    if src == "ball":
        rows, cols = 40, 24 * 200 + 7
        d = synth.leech_matrix(rows, cols, 6, key=(40,))
        coords, scale, tail = d["coords"], d["scale"], d["tail"]
        ids = np.array([leech.class_of(b) for b in coords.reshape(-1, 24)])
    else:
        rows, nb = 30, 50
        cols = 24 * nb
        coords, ids = _all_class_coords(rows, nb, 3)
        scale, tail = synth.fp16_bits(np.ones(rows)), None
    cl = leech.classes()
    want_exc = int(sum(1 for i in ids if i >= 256 or len(set(cl[i]["key"])) > 4))
    blob, n_exc = lvq.expand_lp2x(coords, scale, tail, rows, cols)
    assert n_exc == want_exc and (n_exc > 0)
    assert blob.size == lvq.library().lvq_layout_bytes_lp2x(rows, cols, n_exc)
    u = layout.unpack_lp2x(blob, rows, cols, n_exc)
    assert np.array_equal(u["coords"], coords)
    # a wrong count is refused
    bad = np.empty(lvq.library().lvq_layout_bytes_lp2x(rows, cols, n_exc + 1), dtype=np.uint8)
    assert lvq.library().lvq_expand_lp2x(coords.ctypes.data, scale.ctypes.data,
                                         None if tail is None else tail.ctypes.data, rows, cols,
                                         n_exc + 1, bad.ctypes.data) == lvq.LVQ_E_SHAPE


def test_gemv_rotated_validates_before_launch():
    lib = lvq.library()
    A = 1 << 20
    g = lib.lvq_gemv_rotated
    assert g(A, 4, 4096, None, None, 0, A, A, 1, None) == lvq.LVQ_E_SHAPE    # m = 0
    assert g(A, 4, 4096, None, None, 33, A, A, 1, None) == lvq.LVQ_E_SHAPE   # m > 32
    assert g(A, 4, 4096, None, None, 3, A, A, 1, None) == lvq.LVQ_E_SHAPE    # cols % m
    assert g(A, 4, 24 * 12, None, None, 1, A, A, 1, None) == lvq.LVQ_E_SHAPE  # K = 288
    assert g(A, 4, 16, None, None, 1, A, A, 1, None) == lvq.LVQ_E_SHAPE     # no whole block
    assert g(A, 4, 4096, A + 4, None, 1, A, A, 1, None) == lvq.LVQ_E_ALIGN
    assert g(A, 4, 3 * 1024, None, A + 8, 3, A, A, 1, None) == lvq.LVQ_E_ALIGN
    assert g(A, 4, 4096, None, None, 1, A, A, 0, None) == lvq.LVQ_E_BATCH
    assert g(A, 0, 4096, None, None, 1, A, A, 1, None) == lvq.LVQ_OK


def _direct_words(x):
    blob = lvq.expand_direct(np.asarray(x, np.int8).reshape(1, 1, 24), synth.fp16_bits([1.0]),
                             None, 1, 24)
    return [int(w) for w in blob[:16].view("<u4")]


def test_expand_direct_hand_records():
    # records worked out by hand from the layout rule (|x| = 2e + p; pair P =
    # j // 2 in word P // 3, view v = P % 3, half h = j % 2; e bit f at
    # 1 + f + 16h + 5v, sign at 15 + 16h + 5v, both mod 32)
    x = [4, 4] + [0] * 22                      # e = 2 at j = 0, 1: bits 2 and 18
    assert _direct_words(x) == [0x00040004, 0, 0, 0]
    x = [-3] + [1] * 23                        # p = 1; e = 1 at j = 0, sign bit 15
    assert _direct_words(x) == [0x8003, 0, 0, 0]
    x = [1] * 23 + [-3]                        # j = 23: word 3, v = 2, h = 1
    assert _direct_words(x) == [1, 0, 0, (1 << 27) | (1 << 9)]
    x = [1] * 23 + [13]                        # e = 6: bits 28, 29 (shell 12)
    assert _direct_words(x) == [1, 0, 0, 0x30000000]
    for x in ([4, 4] + [0] * 22, [-3] + [1] * 23, [1] * 23 + [-3], [1] * 23 + [13]):
        assert leech.is_leech(np.array(x))
        blob = lvq.expand_direct(np.array(x, np.int8).reshape(1, 1, 24), synth.fp16_bits([1.0]),
                                 None, 1, 24)
        assert list(layout.unpack_direct(blob, 1, 24)["coords"].reshape(24)) == x


@pytest.mark.parametrize("src", ["ball", "all_classes", "tail_only"])
def test_expand_direct_round_trips_through_the_oracle_unpacker(src):
    if src == "ball":
        rows, cols = 40, 24 * 200 + 7
        d = synth.leech_matrix(rows, cols, 6, key=(41,))
        coords, scale, tail = d["coords"], d["scale"], d["tail"]
    elif src == "all_classes":
        rows, nb = 30, 50
        cols = 24 * nb
        coords, _ = _all_class_coords(rows, nb, 4)
        scale, tail = synth.fp16_bits(np.ones(rows)), None
    else:
        rows, cols = 3, 11
        coords = np.zeros((3, 0, 24), np.int8)
        scale, tail = synth.fp16_bits(np.ones(rows)), synth.fp16_bits(np.ones((rows, 11)))
    blob = lvq.expand_direct(coords, scale, tail, rows, cols)
    assert blob.size == lvq.layout_bytes_direct(rows, cols) == layout.sections_direct(rows, cols)["total"]
    u = layout.unpack_direct(blob, rows, cols)
    assert np.array_equal(u["coords"], coords)
    assert np.array_equal(u["scale"], scale)
    if tail is not None:
        assert np.array_equal(u["tail"], tail)
    # the bits outside p, e and the signs are zero
    used = 1
    for v in range(3):
        for h in range(2):
            for b in (1, 2, 3, 15):
                used |= 1 << ((b + 16 * h + 5 * v) % 32)
    w = u["words"].reshape(-1, 4).astype(np.int64)
    assert np.all(w[:, 0] & ~used & 0xFFFFFFFF == 0)
    assert np.all(w[:, 1:] & ~(used & ~1) & 0xFFFFFFFF == 0)


def test_expand_direct_refusals_and_validation():
    x = np.zeros((2, 3, 24), dtype=np.int8)
    x[1, 2, 0] = 1  # not a lattice point
    with pytest.raises(lvq.LvqError) as e:
        lvq.expand_direct(x, synth.fp16_bits(np.ones(2)), None, 2, 72)
    assert e.value.code == lvq.LVQ_E_NOT_LEECH and e.value.index == (1, 2)
    lib = lvq.library()
    A = 1 << 20
    g = lib.lvq_gemv_direct
    assert g(None, 4, 48, A, A, 1, None) == lvq.LVQ_E_NULL
    assert g(A + 4, 4, 48, A, A, 1, None) == lvq.LVQ_E_ALIGN
    assert g(A, 4, 48, A, A, 0, None) == lvq.LVQ_E_BATCH
    assert g(A, 4, 48, A, A, 5, None) == lvq.LVQ_E_BATCH
    assert g(A, -1, 48, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert g(A, 0, 48, A, A, 1, None) == lvq.LVQ_OK


def _onehot_words(x):
    blob = lvq.expand_onehot(np.asarray(x, np.int8).reshape(1, 1, 24), synth.fp16_bits([1.0]),
                             None, 1, 24)
    off = layout.sections_onehot(1, 24)["codes"]
    return [int(w) for w in blob[off: off + 16].view("<u4")]


def test_expand_onehot_hand_records():
    # worked out by hand from the layout rule: word i marks rank i + 1
    # (coordinate 2P at bit P, 2P + 1 at bit 16 + P); the sign of coordinate
    # 2P (2P + 1) sits in word P // 3 at bit 12 + P % 3 (28 + P % 3)
    cases = [
        ([4, 4] + [0] * 22, [0x00010001, 0, 0, 0]),            # {0, 4}: both rank 1
        ([-3] + [1] * 23, [0x00001001, 0, 0, 0]),               # {1, 3}: rank 1, negative
        ([1] * 23 + [-3], [1 << 27, 0, 0, 1 << 30]),            # pair 11, odd half
        ([1] * 23 + [13], [1 << 27, 0, 0, 0]),                  # shell 12
        ([-3, -7] + [1] * 22, [1 | 1 << 12 | 1 << 28, 1 << 16, 0, 0]),  # {1, 3, 7}
    ]
    for x, want in cases:
        assert leech.is_leech(np.array(x)), x
        assert _onehot_words(x) == want, x
        blob = lvq.expand_onehot(np.array(x, np.int8).reshape(1, 1, 24), synth.fp16_bits([1.0]),
                                 None, 1, 24)
        u = layout.unpack_onehot(blob, 1, 24)
        assert list(u["coords"].reshape(24)) == x
        assert int(u["cls"][0, 0]) == leech.class_of(np.array(x))


@pytest.mark.parametrize("src", ["ball", "all_classes", "tail_only"])
def test_expand_onehot_round_trips_through_the_oracle_unpacker(src):
    if src == "ball":
        rows, cols = 40, 24 * 200 + 7
        d = synth.leech_matrix(rows, cols, 6, key=(43,))
        coords, scale, tail = d["coords"], d["scale"], d["tail"]
    elif src == "all_classes":
        rows, nb = 30, 50
        cols = 24 * nb
        coords, _ = _all_class_coords(rows, nb, 5)
        scale, tail = synth.fp16_bits(np.ones(rows)), None
    else:
        rows, cols = 3, 11
        coords = np.zeros((3, 0, 24), np.int8)
        scale, tail = synth.fp16_bits(np.ones(rows)), synth.fp16_bits(np.ones((rows, 11)))
    blob = lvq.expand_onehot(coords, scale, tail, rows, cols)
    assert blob.size == lvq.layout_bytes_onehot(rows, cols) == layout.sections_onehot(rows, cols)["total"]
    u = layout.unpack_onehot(blob, rows, cols)
    assert np.array_equal(u["coords"], coords)
    assert np.array_equal(u["table"], lvq.class_table())
    assert np.array_equal(u["scale"], scale)
    if tail is not None:
        assert np.array_equal(u["tail"], tail)
    assert np.all(u["words"].astype(np.int64) & 0x80008000 == 0)


def test_gemv_onehot_validates_before_launch():
    lib = lvq.library()
    A = 1 << 20
    g = lib.lvq_gemv_onehot
    assert g(None, 4, 48, A, A, 1, None) == lvq.LVQ_E_NULL
    assert g(A + 4, 4, 48, A, A, 1, None) == lvq.LVQ_E_ALIGN
    assert g(A, 4, 48, A, A, 0, None) == lvq.LVQ_E_BATCH
    assert g(A, -1, 48, A, A, 1, None) == lvq.LVQ_E_SHAPE
    assert g(A, 0, 48, A, A, 1, None) == lvq.LVQ_OK
    x = np.zeros((1, 1, 24), dtype=np.int8)
    x[0, 0, :2] = (2, 2)  # not a lattice point
    with pytest.raises(lvq.LvqError) as e:
        lvq.expand_onehot(x, synth.fp16_bits([1.0]), None, 1, 24)
    assert e.value.code == lvq.LVQ_E_NOT_LEECH and e.value.index == (0, 0)


def test_launch_info_rules_and_validation():
    """The launch the Leech entry points make (nothing is launched): one block
    per lane and a ring of three on rows of two or three 64-block chunks, two
    blocks per lane and a ring of two at 4096 x 12288; LDS = class table + x."""
    lib = lvq.library()
    out = (ctypes.c_int * 5)()
    assert lib.lvq_gemv_launch_info(0, 16, 48, 1, 1, None) == lvq.LVQ_E_NULL
    assert lib.lvq_gemv_launch_info(99, 16, 48, 1, 1, out) == lvq.LVQ_E_SHAPE
    assert lib.lvq_gemv_launch_info(0, 0, 48, 1, 1, out) == lvq.LVQ_E_SHAPE
    assert lib.lvq_gemv_launch_info(0, 16, 48, 5, 1, out) == lvq.LVQ_E_BATCH
    assert lib.lvq_gemv_launch_info(1, 16, 48, 1, 5, out) == lvq.LVQ_E_SHAPE  # 48 % 5
    head = lvq.gemv_launch_info("gemv", 4096, 12288)
    assert (head["blocks_per_lane"], head["ring"]) == (2, 2)
    assert head["lds_bytes"] == 302 * 8 + 12288 * 2
    for rows in (4096, 12288):
        short = lvq.gemv_launch_info("gemv", rows, 4096)
        assert (short["blocks_per_lane"], short["ring"]) == (1, 3)
    # the fused rotation and few rows keep the blocks-per-lane rule
    assert lvq.gemv_launch_info("rotated", 12288, 4096)["ring"] == 2
    assert lvq.gemv_launch_info("gemv", 1024, 4096)["ring"] == 2
    # many waves per SIMD: the blocks per lane that give each wave about four
    # items, not one item per wave; rows of two chunks keep the ring of two
    for rows, cols in ((8192, 6144), (16384, 3072), (32768, 1536)):
        info = lvq.gemv_launch_info("gemv", rows, cols)
        assert (info["blocks_per_lane"], info["ring"]) == (1, 2), (rows, cols)
    wide = lvq.gemv_launch_info("gemv", 2048, 24576)  # two waves per SIMD: largest
    assert wide["blocks_per_lane"] == 4
