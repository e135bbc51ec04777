"""GPU parity of load-time unfolding (48-bit words -> lattice points and gain
bits) and of the shape-gain GEMV, through the C ABI, against the oracle.

Unfolding is integer work: bit-exact against oracle.index.unrank.  The
shape-gain GEMV meets the usual bar (1e-4 of the term-magnitude bound) against
the f64 reconstruction w = s_r * gamma[g] * x.  The served path runs from
random 48-bit words through lvq_unfold, lvq_expand_gain and lvq_gemv_gain.
"""
import numpy as np
import pytest

import synth
from oracle import gemv as og
from oracle import index as oi
from oracle import leech

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_gemv_lvq_amd as lvq  # noqa: E402
from gpu_util import empty, to_dev, to_host  # noqa: E402

GAINS = (0.8125, 1.1875)  # the pages give no levels: two arbitrary fp32 values


def _unfold(words):
    words = np.ascontiguousarray(words, dtype=np.uint64)
    n = words.size
    cd = empty((max(n, 1), 24), np.int8)
    gd = empty((max(n, 16),), np.uint8)
    lvq.unfold(to_dev(words), n, cd, gd)
    return to_host(cd, np.int8)[:n], to_host(gd, np.uint8)[:n]


def test_unfold_random_words_bit_exact():
    rng = np.random.default_rng(2024)
    offs = [int(o) for o in oi.block_offsets()]
    idx = [0, 1, oi.total() - 1, offs[1], offs[1] - 1, offs[4096], offs[4096] - 1, offs[8191]]
    idx += [int(v) for v in rng.integers(0, oi.total(), 3000)]
    gains = rng.integers(0, 2, len(idx))
    words = np.array([oi.word(i, int(g)) for i, g in zip(idx, gains)], dtype=np.uint64)
    coords, gout = _unfold(words)
    want = np.stack([oi.unrank(i) for i in idx])
    assert np.array_equal(coords, want)
    assert np.array_equal(gout, gains.astype(np.uint8))
    print("unfold: %d random words bit-exact" % len(idx), flush=True)


def test_unfold_is_exhaustive_on_shell_2():
    # every minimal vector (the classical construction): ranked on the host,
    # unfolded on the GPU, compared
    from test_oracle_index import _shell2_vectors
    pts = _shell2_vectors()
    assert len(pts) == leech.theta_coefficient(2)
    ranks = lvq.rank(pts)
    assert len(np.unique(ranks)) == len(pts)
    coords, gout = _unfold(ranks)
    assert np.array_equal(coords, pts) and np.all(gout == 0)
    # and a spread sample of those ranks is the oracle's
    for k in range(0, len(pts), 4001):
        assert int(ranks[k]) == oi.rank(pts[k])


def test_unfold_flags_invalid_words():
    bad = np.array([oi.total(), (1 << 47) - 1, 1 << 48, (1 << 63) | 5,
                    oi.word(oi.total() - 1, 1)], dtype=np.uint64)
    coords, gout = _unfold(bad)
    assert list(gout) == [0xFF, 0xFF, 0xFF, 0xFF, 1]
    assert np.all(coords[:4] == 0)
    assert np.array_equal(coords[4], oi.unrank(oi.total() - 1))


@pytest.mark.parametrize("rows,cols,batch", [(4096, 12288, 1), (4096, 4096, 4), (130, 24 * 65 + 7, 3),
                                             (257, 24 * 129, 2)])
def test_gain_gemv(rows, cols, batch):
    d = synth.leech_matrix(rows, cols, 3, key=(rows, cols, 9))
    g = np.random.default_rng(rows + cols).integers(0, 2, (rows, cols // 24)).astype(np.uint8)
    blob = lvq.expand_gain(d["coords"], g, d["scale"], d["tail"], rows, cols)
    x = synth.activations(cols, batch, 3, rows=rows)
    yd = empty((batch, rows), np.float32)
    lvq.gemv_gain(to_dev(blob), rows, cols, GAINS[0], GAINS[1], to_dev(x), yd, batch)
    w = oi.shape_gain_weights(d["coords"], g, d["scale"], GAINS, d["tail"], cols)
    y64, bound = og.gemv(w, x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    print("gain gemv %dx%d b%d: max |err| / (1e-4 * bound) = %.3g" % (rows, cols, batch, r),
          flush=True)
    assert r <= 1.0


def test_served_path_from_48_bit_words():
    """Random words -> unfold (GPU) -> expand_gain (host) -> gain GEMV (GPU)."""
    rows, nb, tau, batch = 48, 40, 5, 2
    cols = 24 * nb + tau
    rng = np.random.default_rng(77)
    idx = rng.integers(0, oi.total(), rows * nb)
    gbits = rng.integers(0, 2, rows * nb)
    words = np.array([oi.word(int(i), int(b)) for i, b in zip(idx, gbits)], dtype=np.uint64)
    coords, gout = _unfold(words)
    scale = synth.fp16_bits(np.abs(rng.standard_normal(rows)) * 0.01)
    tail = synth.fp16_bits(rng.standard_normal((rows, tau)) * 0.02)
    blob = lvq.expand_gain(coords.reshape(rows, nb, 24), gout.reshape(rows, nb), scale, tail,
                           rows, cols)
    x = synth.activations(cols, batch, 3, key=(77,))
    yd = empty((batch, rows), np.float32)
    lvq.gemv_gain(to_dev(blob), rows, cols, GAINS[0], GAINS[1], to_dev(x), yd, batch)
    pts = np.stack([oi.unrank(int(i)) for i in idx]).reshape(rows, nb, 24)
    w = oi.shape_gain_weights(pts, gbits.reshape(rows, nb), scale, GAINS, tail, cols)
    y64, bound = og.gemv(w, x)
    assert og.check(to_host(yd, np.float32), y64, bound) <= 1.0
