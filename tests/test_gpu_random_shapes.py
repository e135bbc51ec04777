"""GPU parity over a seeded list of random shapes, through the C ABI, against
the f64 oracle: rows 1..2100, 0..400 whole blocks with and without a tail,
batch 1..4, blocks drawn uniformly over the 301 classes, from the workload's
shells 2..6, or from the whole ball with P(m) ~ 2^-m.
Every Leech entry point that reads a matrix takes the same matrix: LP3, the
shape-gain mode with both gain levels 1 (its arithmetic then equals LP3's
but for the partial sums per word), LP2X, the direct and one-hot layouts.
The shapes sweep the launch choices (blocks per lane 1..4, one to many
chunks per row, workgroups of 256..1024 threads) that fixed cases visit
only a few of."""
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


def _shapes():
    rng = np.random.default_rng(20261202)
    out = []
    for i in range(24):
        rows = int(rng.choice([1, 7, 64, 130, 257, 511, 1024, 2100]))
        nb = int(rng.integers(0, 401))
        tau = int(rng.choice([0, 0, 1, 5, 16, 23]))
        if nb == 0 and tau == 0:
            tau = 7
        batch = int(rng.integers(1, 5))
        dist = str(rng.choice(["classes", "m2to6", "ball"]))
        out.append((i, rows, nb, tau, batch, dist))
    return out


def _matrix(rows, nb, tau, dist, seed):
    if dist != "classes":
        return synth.leech_matrix(rows, 24 * nb + tau, 3 if dist == "m2to6" else 6, key=(seed,))
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, leech.NUM_CLASSES, rows * nb)
    cl = leech.classes()
    coords = np.zeros((rows * nb, 24), dtype=np.int8)
    for cid in np.unique(ids):
        sel = np.nonzero(ids == cid)[0]
        if cid:
            coords[sel] = synth.sample_class(cl[cid]["key"], sel.size, rng)
    coords = coords.reshape(rows, nb, 24)
    return {"coords": coords,
            "scale": synth.fp16_bits(np.abs(rng.standard_normal(rows)) * 0.02),
            "tail": synth.fp16_bits(rng.standard_normal((rows, tau)) * 0.02)}


@pytest.mark.parametrize("case", _shapes(), ids=lambda c: "s%d-%dx%d+%d-b%d-%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5]))
def test_every_layout_on_random_shapes(case):
    i, rows, nb, tau, batch, dist = case
    cols = 24 * nb + tau
    d = _matrix(rows, nb, tau, dist, seed=1000 + i)
    x = synth.activations(cols, batch, 3, key=(i, 17))
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x)
    xd = to_dev(x)
    args = (d["coords"], d["scale"], d["tail"], rows, cols)
    runs = {
        "lp3": lambda y: lvq.gemv(to_dev(lvq.expand(*args)), rows, cols, xd, y, batch),
        "gain": lambda y: lvq.gemv_gain(
            to_dev(lvq.expand_gain(d["coords"], np.zeros((rows, nb), np.uint8), d["scale"],
                                   d["tail"], rows, cols)), rows, cols, 1.0, 1.0, xd, y, batch),
        "direct": lambda y: lvq.gemv_direct(to_dev(lvq.expand_direct(*args)), rows, cols, xd, y,
                                            batch),
        "onehot": lambda y: lvq.gemv_onehot(to_dev(lvq.expand_onehot(*args)), rows, cols, xd, y,
                                            batch),
    }
    blob_x, n_exc = lvq.expand_lp2x(*args)
    runs["lp2x"] = lambda y: lvq.gemv_lp2x(to_dev(blob_x), rows, cols, n_exc, xd, y, batch)
    worst = 0.0
    for name, run in runs.items():
        yd = empty((batch, rows), np.float32)
        run(yd)
        r = og.check(to_host(yd, np.float32), y64, bound)
        worst = max(worst, r)
        assert r <= 1.0, name
    print("random shape %d (%dx%d, b%d, %s): worst ratio %.3g" % (
        i, rows, cols, batch, dist, worst), flush=True)
