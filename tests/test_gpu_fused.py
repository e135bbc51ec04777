"""GPU parity of the fused multi-projection launch and the no-weights control,
through the C ABI.

lvq_gemv_fused runs several Leech matrices that share x (q, k, v; gate, up) in
one launch.  Every output is checked against the f64 oracle at the usual bar
and, bit for bit, against separate lvq_gemv calls: a row's sum does not depend
on the launch geometry.  lvq_gemv_noweights makes lvq_gemv's launch without
reading weights; its output is +0.0 exactly.
"""
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

SENTINEL = np.float32(-12345.5)
PAD = 64  # floats past each output that no call may touch


def _all_class_matrix(rows, nb, tau, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, leech.NUM_CLASSES, rows * nb)
    cl = leech.classes()
    coords = np.zeros((rows * nb, 24), dtype=np.int8)
    for cid in np.unique(ids):
        sel = np.nonzero(ids == cid)[0]
        if cid:
            coords[sel] = synth.sample_class(cl[cid]["key"], sel.size, rng)
    return {"coords": coords.reshape(rows, nb, 24),
            "scale": synth.fp16_bits(np.abs(rng.standard_normal(rows)) * 0.02),
            "tail": synth.fp16_bits(rng.standard_normal((rows, tau)) * 0.02),
            "rows": rows, "cols": 24 * nb + tau}


def _padded_out(n):
    return to_dev(np.full(n + PAD, SENTINEL, dtype=np.float32))


def _run_both(mats, x_bits, batch):
    """Fused launch and separate launches over the same device blobs."""
    cols = mats[0]["cols"]
    blobs = [to_dev(lvq.expand(d["coords"], d["scale"], d["tail"], d["rows"], cols))
             for d in mats]
    xd = to_dev(x_bits)
    yf = [_padded_out(batch * d["rows"]) for d in mats]
    ys = [_padded_out(batch * d["rows"]) for d in mats]
    lvq.gemv_fused(blobs, [d["rows"] for d in mats], cols, xd, yf, batch)
    for b, d, y in zip(blobs, mats, ys):
        lvq.gemv(b, d["rows"], cols, xd, y, batch)
    out = []
    for d, a, b in zip(mats, yf, ys):
        n = batch * d["rows"]
        fa, fb = to_host(a, np.float32), to_host(b, np.float32)
        assert np.all(fa[n:] == SENTINEL), "fused launch wrote past an output"
        assert np.array_equal(fa[:n].view(np.uint32), fb[:n].view(np.uint32)), \
            "fused and separate results differ"
        out.append(fa[:n].reshape(batch, d["rows"]))
    return out


def _oracle_check(d, x_bits, y, name):
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], d["cols"])
    y64, bound = og.gemv(w, x_bits)
    r = og.check(y, y64, bound)
    print("%s %dx%d: max |err| / (1e-4 * bound) = %.3g" % (name, d["rows"], d["cols"], r),
          flush=True)
    assert r <= 1.0


@pytest.mark.parametrize("batch", [1, 4])
def test_fused_qwen3_8b_qkv_and_gate_up(batch):
    """Layer 0 of the 8B stack: q (4096), k (1024), v (1024) over the layer
    input in one launch; gate and up (12288 each) over one x in another."""
    q, k, v, _, gate, up, _ = [synth.qwen3_8b_matrix(0, m)
                               for m in range(len(synth.QWEN3_8B_MATRICES))]
    h = synth.activations(4096, batch, 5, key=(0, batch))
    yq, yk, yv = _run_both([q, k, v], h, batch)
    for d, y, name in ((q, yq, "q"), (k, yk, "k"), (v, yv, "v")):
        _oracle_check(d, h, y, "fused %s b%d" % (name, batch))
    xg = synth.activations(4096, batch, 5, key=(1, batch))
    yg, yu = _run_both([gate, up], xg, batch)
    _oracle_check(gate, xg, yg, "fused gate b%d" % batch)
    _oracle_check(up, xg, yu, "fused up b%d" % batch)


@pytest.mark.parametrize("rows,nb,tau,batch", [
    ((1,), 1, 0, 1),
    ((300, 5), 170, 16, 2),
    ((7, 0, 129, 64), 65, 7, 3),       # a matrix with no rows in the middle
    ((33, 257, 1, 130), 129, 0, 4),
    ((40, 41, 42), 600, 5, 1),         # rows longer than one chunk
    ((3, 9), 0, 23, 2),                # tails only
    ((1000, 1, 17, 500), 40, 11, 1),
])
def test_fused_ragged(rows, nb, tau, batch):
    mats = [_all_class_matrix(r, nb, tau, seed=1000 * r + 7 * i + nb)
            for i, r in enumerate(rows)]
    x = synth.activations(24 * nb + tau, batch, 3, key=(len(rows), nb, tau))
    ys = _run_both(mats, x, batch)
    for i, (d, y) in enumerate(zip(mats, ys)):
        if d["rows"]:
            _oracle_check(d, x, y, "fused ragged m%d b%d" % (i, batch))


def test_fused_zero_columns_and_rows():
    ys = [to_dev(np.full(2 * r, 5.0, dtype=np.float32)) for r in (3, 4)]
    blobs = [to_dev(lvq.expand(np.zeros((r, 0, 24), np.int8), np.zeros(r, np.uint16), None, r, 0))
             for r in (3, 4)]
    lvq.gemv_fused(blobs, [3, 4], 0, to_dev(np.zeros(8, np.uint16)), ys, 2)
    for y in ys:
        assert np.all(to_host(y, np.float32) == 0)
    # no rows at all: nothing is launched
    lvq.gemv_fused(blobs, [0, 0], 4096, to_dev(np.zeros(4096, np.uint16)), ys, 1)


@pytest.mark.parametrize("rows,cols,batch", [(4096, 12288, 1), (12288, 4096, 4),
                                             (4096, 4096, 2), (300, 1000, 3), (5, 23, 1)])
def test_noweights_reads_no_weights(rows, cols, batch):
    d = synth.leech_matrix(rows, cols, 3) if cols >= 24 else _all_class_matrix(rows, 0, cols, 3)
    blob = to_dev(lvq.expand(d["coords"], d["scale"], d["tail"], rows, cols))
    x = to_dev(synth.activations(cols, batch, 3, key=(rows, cols)))
    y = _padded_out(batch * rows)
    lvq.gemv_noweights(blob, rows, cols, x, y, batch)
    got = to_host(y, np.float32)
    n = batch * rows
    assert np.all(got[n:] == SENTINEL)
    assert np.all(got[:n].view(np.uint32) == 0), "no-weights output is not +0.0"
    # the same blob through the real kernel gives a nonzero result
    yr = empty((batch, rows), np.float32)
    lvq.gemv(blob, rows, cols, x, yr, batch)
    assert np.any(to_host(yr, np.float32) != 0)
