"""GPU parity of the compact and alternative layouts through the C ABI: LP2
(two rank planes, class inside the record) against the f64 oracle, and bit for
bit against the LP3 kernel on the same matrix (both decode to the same fp16
values and sum in the same column order); LP2X with its side channel; the
table-free direct layout against the oracle, and its results independent of
the batch size (so of the blocks per lane the launch picks); the one-hot
layout against the oracle and bit for bit against the direct layout."""
import numpy as np
import pytest

import synth
from oracle import gemv as og
from oracle import leech

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_gemv_lvq_amd as lvq  # noqa: E402
from gpu_util import empty, to_dev, to_host  # noqa: E402


def _both(d, rows, cols, x, batch):
    y2 = empty((batch, rows), np.float32)
    y3 = empty((batch, rows), np.float32)
    lvq.gemv_lp2(to_dev(lvq.expand_lp2(d["coords"], d["scale"], d["tail"], rows, cols)), rows,
                 cols, to_dev(x), y2, batch)
    lvq.gemv(to_dev(lvq.expand(d["coords"], d["scale"], d["tail"], rows, cols)), rows, cols,
             to_dev(x), y3, batch)
    return to_host(y2, np.float32), to_host(y3, np.float32)


@pytest.mark.parametrize("rows,cols,cfg,batch", [
    (4096, 12288, 4, 1), (4096, 12288, 4, 4), (12288, 4096, 3, 1), (4096, 4096, 3, 2),
    (1536, 1536, 1, 1), (130, 24 * 65 + 7, 3, 3), (257, 24 * 129, 4, 1), (5, 23, 3, 1),
])
def test_lp2_gemv(rows, cols, cfg, batch):
    d = synth.leech_matrix(rows, cols, cfg, key=(rows, cols, cfg))
    x = synth.activations(cols, batch, cfg, rows=rows)
    y2, y3 = _both(d, rows, cols, x, batch)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    r = og.check(y2, y64, bound)
    print("lp2 %dx%d cfg%d b%d: max |err| / (1e-4 * bound) = %.3g" % (rows, cols, cfg, batch, r),
          flush=True)
    assert r <= 1.0
    assert np.array_equal(y2.view(np.uint32), y3.view(np.uint32))


def test_lp2_gemv_every_eligible_class():
    rng = np.random.default_rng(12)
    ok = [c for c in leech.classes() if c["id"] < 256 and len(set(c["key"])) <= 4]
    rows, nb = 64, 70
    ids = rng.choice([c["id"] for c in ok], rows * nb)
    cl = leech.classes()
    coords = np.zeros((rows * nb, 24), dtype=np.int8)
    for cid in np.unique(ids):
        sel = np.nonzero(ids == cid)[0]
        if cid:
            coords[sel] = synth.sample_class(cl[cid]["key"], sel.size, rng)
    d = {"coords": coords.reshape(rows, nb, 24),
         "scale": synth.fp16_bits(np.abs(rng.standard_normal(rows)) * 0.02),
         "tail": synth.fp16_bits(rng.standard_normal((rows, 9)) * 0.02)}
    cols = 24 * nb + 9
    x = synth.activations(cols, 2, 3, key=(12,))
    y2, y3 = _both(d, rows, cols, x, 2)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    assert og.check(y2, y64, bound) <= 1.0
    assert np.array_equal(y2.view(np.uint32), y3.view(np.uint32))


@pytest.mark.parametrize("rows,cols,batch", [(4096, 12288, 1), (4096, 4096, 4), (300, 24 * 170 + 5, 2)])
def test_lp2x_gemv_whole_ball(rows, cols, batch):
    d = synth.leech_matrix(rows, cols, 6, key=(rows, cols, 6))
    blob, n_exc = lvq.expand_lp2x(d["coords"], d["scale"], d["tail"], rows, cols)
    assert n_exc > 0
    x = synth.activations(cols, batch, 6, rows=rows)
    yd = empty((batch, rows), np.float32)
    lvq.gemv_lp2x(to_dev(blob), rows, cols, n_exc, to_dev(x), yd, batch)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    print("lp2x %dx%d b%d (%d side-channel blocks): max |err| / (1e-4 * bound) = %.3g"
          % (rows, cols, batch, n_exc, r), flush=True)
    assert r <= 1.0


def test_lp2x_gemv_every_class():
    rng = np.random.default_rng(31)
    rows, nb = 96, 40
    ids = rng.integers(0, leech.NUM_CLASSES, rows * nb)
    cl = leech.classes()
    coords = np.zeros((rows * nb, 24), dtype=np.int8)
    for cid in np.unique(ids):
        sel = np.nonzero(ids == cid)[0]
        if cid:
            coords[sel] = synth.sample_class(cl[cid]["key"], sel.size, rng)
    coords = coords.reshape(rows, nb, 24)
    cols = 24 * nb + 3
    scale = synth.fp16_bits(np.abs(rng.standard_normal(rows)) * 0.02)
    tail = synth.fp16_bits(rng.standard_normal((rows, 3)) * 0.02)
    blob, n_exc = lvq.expand_lp2x(coords, scale, tail, rows, cols)
    x = synth.activations(cols, 3, 6, key=(31,))
    yd = empty((3, rows), np.float32)
    lvq.gemv_lp2x(to_dev(blob), rows, cols, n_exc, to_dev(x), yd, 3)
    w = og.leech_weights(coords, scale, tail, cols)
    y64, bound = og.gemv(w, x)
    assert og.check(to_host(yd, np.float32), y64, bound) <= 1.0


def _direct(d, rows, cols, x, batch):
    yd = empty((batch, rows), np.float32)
    lvq.gemv_direct(to_dev(lvq.expand_direct(d["coords"], d["scale"], d["tail"], rows, cols)),
                    rows, cols, to_dev(x), yd, batch)
    return to_host(yd, np.float32)


@pytest.mark.parametrize("rows,cols,cfg,batch", [
    (4096, 12288, 4, 1), (4096, 12288, 6, 4), (12288, 4096, 3, 1), (4096, 4096, 6, 2),
    (1536, 1536, 1, 3), (130, 24 * 65 + 7, 3, 3), (257, 24 * 129, 6, 1), (5, 23, 3, 1),
])
def test_direct_gemv(rows, cols, cfg, batch):
    d = synth.leech_matrix(rows, cols, cfg, key=(rows, cols, cfg, 16))
    x = synth.activations(cols, batch, cfg, rows=rows)
    y = _direct(d, rows, cols, x, batch)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    r = og.check(y, y64, bound)
    print("direct %dx%d cfg%d b%d: max |err| / (1e-4 * bound) = %.3g" % (rows, cols, cfg, batch, r),
          flush=True)
    assert r <= 1.0
    if batch > 1:
        y1 = _direct(d, rows, cols, np.ascontiguousarray(x[:1]), 1)
        assert np.array_equal(y[:1].view(np.uint32), y1.view(np.uint32))


def test_direct_gemv_every_class():
    rng = np.random.default_rng(33)
    rows, nb = 96, 40
    ids = rng.integers(0, leech.NUM_CLASSES, rows * nb)
    cl = leech.classes()
    coords = np.zeros((rows * nb, 24), dtype=np.int8)
    for cid in np.unique(ids):
        sel = np.nonzero(ids == cid)[0]
        if cid:
            coords[sel] = synth.sample_class(cl[cid]["key"], sel.size, rng)
    cols = 24 * nb + 3
    d = {"coords": coords.reshape(rows, nb, 24),
         "scale": synth.fp16_bits(np.abs(rng.standard_normal(rows)) * 0.02),
         "tail": synth.fp16_bits(rng.standard_normal((rows, 3)) * 0.02)}
    x = synth.activations(cols, 4, 6, key=(33,))
    y = _direct(d, rows, cols, x, 4)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    assert og.check(y, y64, bound) <= 1.0


def _onehot(d, rows, cols, x, batch):
    yd = empty((batch, rows), np.float32)
    lvq.gemv_onehot(to_dev(lvq.expand_onehot(d["coords"], d["scale"], d["tail"], rows, cols)),
                    rows, cols, to_dev(x), yd, batch)
    return to_host(yd, np.float32)


@pytest.mark.parametrize("rows,cols,cfg,batch", [
    (4096, 12288, 4, 1), (4096, 12288, 6, 4), (12288, 4096, 3, 1), (4096, 4096, 6, 2),
    (1536, 1536, 1, 3), (130, 24 * 65 + 7, 3, 3), (257, 24 * 129, 6, 1), (5, 23, 3, 1),
])
def test_onehot_gemv(rows, cols, cfg, batch):
    """Against the oracle, and bit for bit against the direct layout: both
    decode to the same fp16 pairs and sum them in the same order."""
    d = synth.leech_matrix(rows, cols, cfg, key=(rows, cols, cfg, 17))
    x = synth.activations(cols, batch, cfg, rows=rows)
    y = _onehot(d, rows, cols, x, batch)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    r = og.check(y, y64, bound)
    print("onehot %dx%d cfg%d b%d: max |err| / (1e-4 * bound) = %.3g" % (rows, cols, cfg, batch, r),
          flush=True)
    assert r <= 1.0
    assert np.array_equal(y.view(np.uint32), _direct(d, rows, cols, x, batch).view(np.uint32))


def test_onehot_gemv_every_class():
    rng = np.random.default_rng(34)
    rows, nb = 96, 40
    ids = rng.integers(0, leech.NUM_CLASSES, rows * nb)
    cl = leech.classes()
    coords = np.zeros((rows * nb, 24), dtype=np.int8)
    for cid in np.unique(ids):
        sel = np.nonzero(ids == cid)[0]
        if cid:
            coords[sel] = synth.sample_class(cl[cid]["key"], sel.size, rng)
    cols = 24 * nb + 5
    d = {"coords": coords.reshape(rows, nb, 24),
         "scale": synth.fp16_bits(np.abs(rng.standard_normal(rows)) * 0.02),
         "tail": synth.fp16_bits(rng.standard_normal((rows, 5)) * 0.02)}
    x = synth.activations(cols, 3, 6, key=(34,))
    y = _onehot(d, rows, cols, x, 3)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    assert og.check(y, y64, bound) <= 1.0


def test_lp2x_without_side_channel_reads_as_lp2():
    # shells 2..6 fit LP2 everywhere: no entries, and the LP2X blob's LP2 part
    # is the LP2 blob, so the results are the LP2 kernel's bit for bit
    rows, cols, batch = 300, 24 * 170 + 5, 3
    d = synth.leech_matrix(rows, cols, 3, key=(rows, cols, 71))
    blob, n_exc = lvq.expand_lp2x(d["coords"], d["scale"], d["tail"], rows, cols)
    assert n_exc == 0
    x = synth.activations(cols, batch, 3, key=(71,))
    yx = empty((batch, rows), np.float32)
    lvq.gemv_lp2x(to_dev(blob), rows, cols, 0, to_dev(x), yx, batch)
    y2 = empty((batch, rows), np.float32)
    lvq.gemv_lp2(to_dev(lvq.expand_lp2(d["coords"], d["scale"], d["tail"], rows, cols)), rows,
                 cols, to_dev(x), y2, batch)
    assert np.array_equal(to_host(yx, np.float32).view(np.uint32),
                          to_host(y2, np.float32).view(np.uint32))
