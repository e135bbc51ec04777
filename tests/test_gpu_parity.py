"""GPU parity: every kernel, through the C ABI, against the f64 oracle.

Bar: decoded integer coordinates bit-exact; every GEMV output within
|y - y_f64| <= 1e-4 * sum_c |w_rc x_c| (rows whose bound is 0 exactly 0).
Sizes span several tiles and ragged tails; the largest cases are the
workload shapes (1536^2, 4096^2, 12288x4096, 4096x12288), run in the launch
configuration the bench times.
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

TOL = og.REL_TOL


def _report(name, ratio):
    print("%s: max |err| / (1e-4 * bound) = %.3g" % (name, ratio), flush=True)


# ---------------------------------------------------------------- Leech helpers

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


def _leech_gpu(d, x_bits, batch):
    rows, cols = d["rows"], d["cols"]
    blob = lvq.expand(d["coords"], d["scale"], d["tail"], rows, cols)
    bd = to_dev(blob)
    xd = to_dev(x_bits)
    yd = empty((batch, rows), np.float32)
    lvq.gemv(bd, rows, cols, xd, yd, batch)
    return to_host(yd, np.float32), bd


def _leech_parity(d, batch, cfg, name):
    x = synth.activations(d["cols"], batch, cfg, rows=d["rows"])
    y, _ = _leech_gpu(d, x, batch)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], d["cols"])
    y64, bound = og.gemv(w, x)
    r = og.check(y, y64, bound)
    _report(name, r)
    assert r <= 1.0
    return y


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("rows,cols,cfg", [(1536, 1536, 1), (300, 4096, 3)])
def test_decode_bit_exact(rows, cols, cfg):
    d = synth.leech_matrix(rows, cols, cfg)
    blob = lvq.expand(d["coords"], d["scale"], d["tail"], rows, cols)
    out = empty((rows, cols // 24, 24), np.int8)
    lvq.decode(to_dev(blob), rows, cols, out)
    got = to_host(out, np.int8)
    assert np.array_equal(got, d["coords"])
    # bijection: the decoded points re-expand to the same blob
    again = lvq.expand(got, d["scale"], d["tail"], rows, cols)
    assert np.array_equal(again, blob)


def test_decode_every_class_bit_exact():
    d = _all_class_matrix(64, 40, 0, seed=21)
    blob = lvq.expand(d["coords"], d["scale"], d["tail"], 64, d["cols"])
    out = empty((64, 40, 24), np.int8)
    lvq.decode(to_dev(blob), 64, d["cols"], out)
    assert np.array_equal(to_host(out, np.int8), d["coords"])


# ---------------------------------------------------------------- Leech GEMV

@pytest.mark.parametrize("rows,cols,cfg,batch", [
    (1536, 1536, 1, 1),
    (4096, 4096, 3, 1),
    (4096, 4096, 3, 4),
    (12288, 4096, 3, 1),
    (12288, 4096, 3, 4),
    (4096, 12288, 4, 1),
    (4096, 12288, 4, 4),
])
def test_leech_gemv_workloads(rows, cols, cfg, batch):
    d = synth.leech_matrix(rows, cols, cfg)
    _leech_parity(d, batch, cfg, "leech %dx%d cfg%d b%d" % (rows, cols, cfg, batch))


@pytest.mark.parametrize("rows,nb,tau,batch", [
    (1, 1, 0, 1), (3, 0, 23, 1), (5, 1, 1, 2), (64, 170, 16, 1), (130, 65, 7, 3),
    (257, 129, 0, 4), (33, 200, 5, 1),
    (40, 600, 5, 2), (17, 1024, 0, 1), (300, 520, 3, 1),  # rows longer than one chunk
    (64, 682, 16, 4), (100, 2730, 16, 1),  # batch x cols at its limit, 65,536
    (8193, 171, 5, 3), (8195, 130, 0, 4),  # many rows per wave at batch 3 and 4, odd counts
])
def test_leech_gemv_ragged_and_full_ball(rows, nb, tau, batch):
    d = _all_class_matrix(rows, nb, tau, seed=rows * 1000 + nb)
    _leech_parity(d, batch, 3, "leech all-class %dx%d+%d b%d" % (rows, nb, tau, batch))


def test_leech_gemv_exact_special_cases():
    rows, cols = 96, 24 * 70 + 10
    d = _all_class_matrix(rows, 70, 10, seed=5)
    d["scale"][3] = 0            # row 3: tail only
    d["coords"][4] = 0           # row 4: all blocks zero ...
    d["tail"][4] = 0             # ... and zero tail: bound 0, y must be exactly 0
    s = og.f16(d["scale"])
    for c in (0, 23, 24 * 37 + 5, 24 * 70 - 1):
        x = np.zeros((1, cols), dtype=np.float16)
        x[0, c] = 1.0
        y, _ = _leech_gpu(d, x.view(np.uint16), 1)
        k, j = divmod(c, 24)
        assert np.array_equal(y[0], (s * d["coords"][:, k, j]).astype(np.float32))
    x = synth.activations(cols, 2, 3, rows=rows)
    y, _ = _leech_gpu(d, x, 2)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    assert og.check(y, y64, bound) <= 1.0
    assert np.all(y[:, 4] == 0)


def test_leech_gemv_deterministic_and_degenerate():
    d = synth.leech_matrix(512, 4096, 3)
    x = synth.activations(4096, 1, 3)
    y1, bd = _leech_gpu(d, x, 1)
    y2, _ = _leech_gpu(d, x, 1)
    assert np.array_equal(y1, y2)
    # zero columns: y is all zeros; zero rows: nothing to do
    yd = to_dev(np.full((2, 7), 5.0, dtype=np.float32))
    lvq.gemv(to_dev(lvq.expand(np.zeros((7, 0, 24), np.int8), np.zeros(7, np.uint16), None, 7, 0)),
             7, 0, to_dev(np.zeros(16, np.uint16)), yd, 2)
    assert np.all(to_host(yd, np.float32) == 0)
    lvq.gemv(bd, 0, 4096, to_dev(x), yd, 1)


# ---------------------------------------------------------------- fp16 control

@pytest.mark.parametrize("rows,cols,batch", [(4096, 4096, 1), (4096, 12288, 1), (300, 1000, 3),
                                             (65, 8, 4)])
def test_fp16_gemv(rows, cols, batch):
    wb = synth.dense_matrix(rows, cols)
    x = synth.activations(cols, batch, 2, rows=rows)
    yd = empty((batch, rows), np.float32)
    lvq.fp16_gemv(to_dev(wb), rows, cols, to_dev(x), yd, batch)
    y64, bound = og.gemv(og.fp16_weights(wb, rows, cols), x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    _report("fp16 %dx%d b%d" % (rows, cols, batch), r)
    assert r <= 1.0


# ---------------------------------------------------------------- BPDQ

@pytest.mark.parametrize("rows,cols,batch", [(4096, 4096, 1), (4096, 4096, 4), (33, 256, 1),
                                             (100, 4352, 2), (300, 1024, 3),
                                             # 64 quarters per workgroup row
                                             (4096, 12288, 1), (12288, 4096, 4)])
def test_bpdq_gemv(rows, cols, batch):
    d = synth.bpdq_matrix(rows, cols)
    x = synth.activations(cols, batch, 2, rows=rows)
    yd = empty((batch, rows), np.float32)
    lvq.bpdq_gemv(to_dev(d["codes"]), to_dev(d["coeffs"]), rows, cols, to_dev(x), yd, batch)
    y64, bound = og.gemv(og.bpdq_weights(d["codes"], d["coeffs"], rows, cols), x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    _report("bpdq %dx%d b%d" % (rows, cols, batch), r)
    assert r <= 1.0


# ---------------------------------------------------------------- trellis

@pytest.mark.parametrize("rows,cols,batch", [(4096, 12288, 1), (16, 256, 1), (70, 512, 2),
                                             (9, 3072, 4)])
def test_trellis_gemv(rows, cols, batch):
    d = synth.trellis_matrix(rows, cols)
    x = synth.activations(cols, batch, 4, rows=rows)
    yd = empty((batch, rows), np.float32)
    lvq.trellis_gemv(to_dev(d["bits"]), to_dev(d["table"]), to_dev(d["scale"]), rows, cols,
                     to_dev(x), yd, batch)
    w = og.trellis_weights(d["bits"], d["table"], d["scale"], rows, cols)
    y64, bound = og.gemv(w, x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    _report("trellis %dx%d b%d" % (rows, cols, batch), r)
    assert r <= 1.0


# ---------------------------------------------------------------- streaming reference

@pytest.mark.parametrize("nbytes", [4, 20, 4096, 1 << 20, (29368320 // 16) * 16 + 12])
def test_stream_read_checksum(nbytes):
    words = np.random.default_rng(nbytes).integers(0, 1 << 32, nbytes // 4, dtype=np.uint64)
    words = words.astype(np.uint32)
    sink = to_dev(np.zeros(lvq.STREAM_SINK_WORDS, dtype=np.uint32))
    lvq.stream_read(to_dev(words), nbytes, sink)
    got = np.bitwise_xor.reduce(to_host(sink, np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))
