"""GPU parity of the activation rotation y = (H kron Q)(S x), through the C
ABI, against the f64 oracle.

Bar: |y - y64| <= ulp16(y64) + 1e-5 * bound per element (the device rounds an
fp32 result to fp16 once).  Widths are the Qwen3 family's projection inputs
(2560 = 5 x 512, 4096, 5120 = 5 x 1024, 9728 = 19 x 512, 12288 = 3 x 4096,
17408 = 17 x 1024, 25600 = 25 x 1024) plus ragged and degenerate cases.
"""
import numpy as np
import pytest

import synth
from oracle import rotate as orot

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_gemv_lvq_amd as lvq  # noqa: E402
from gpu_util import empty, to_dev, to_host  # noqa: E402


def _orthogonal(rng, m):
    a, _ = np.linalg.qr(rng.standard_normal((m, m)))
    return a.astype(np.float32)


def _case(n, m, batch, seed, signs=True, q=True, scale=1.0):
    rng = np.random.default_rng(seed)
    x = synth.fp16_bits(rng.standard_normal((batch, n)) * scale)
    words = (rng.integers(0, 1 << 32, max(1, (n + 31) // 32), dtype=np.uint64).astype(np.uint32)
             if signs else None)
    qm = _orthogonal(rng, m) if q else None
    return x, words, qm


def _run(x, words, qm, n, m, batch, inplace=False):
    xd = to_dev(x)
    yd = xd if inplace else empty((batch, n), np.uint16)
    lvq.rotate(xd, n, m, None if words is None else to_dev(words),
               None if qm is None else to_dev(qm), yd, batch)
    return to_host(yd, np.uint16)


@pytest.mark.parametrize("n,m,batch", [
    (4096, 1, 1), (4096, 1, 4), (12288, 3, 1), (12288, 3, 4), (2560, 5, 2), (5120, 5, 1),
    (9728, 19, 1), (17408, 17, 1), (25600, 25, 1), (32768, 1, 2), (6144, 3, 3),
])
def test_rotate_widths(n, m, batch):
    x, words, qm = _case(n, m, batch, seed=n + m + batch)
    y = _run(x, words, qm, n, m, batch)
    y64, bound = orot.rotate(x, n, m, words, None if qm is None else qm.astype(np.float64))
    r = orot.rotate_check(y, y64, bound)
    print("rotate n=%d m=%d b%d: max |err| / tol = %.3g" % (n, m, batch, r), flush=True)
    assert r <= 1.0


@pytest.mark.parametrize("n,m,signs,q", [
    (1, 1, False, False), (2, 1, True, False), (8, 1, True, True), (3, 3, True, True),
    (24, 3, False, True), (48, 3, True, False), (7 * 64, 7, True, True), (31 * 2, 31, True, True),
    (32 * 16, 32, False, True), (40, 5, True, True), (1 << 14, 1, False, False),
])
def test_rotate_ragged_and_degenerate(n, m, signs, q):
    x, words, qm = _case(n, m, 2, seed=7 * n + m, signs=signs, q=q)
    y = _run(x, words, qm, n, m, 2)
    y64, bound = orot.rotate(x, n, m, words, None if qm is None else qm.astype(np.float64))
    assert orot.rotate_check(y, y64, bound) <= 1.0


def test_rotate_in_place_and_exact_cases():
    n = 1024
    x, words, _ = _case(n, 1, 3, seed=5)
    y_sep = _run(x, words, None, n, 1, 3)
    y_in = _run(x, words, None, n, 1, 3, inplace=True)
    assert np.array_equal(y_sep, y_in)
    # a unit vector maps to +-1/32 exactly; a constant vector to one spike
    e = np.zeros((1, n), dtype=np.float16)
    e[0, 37] = 1.0
    y = _run(e.view(np.uint16), None, None, n, 1, 1).view(np.float16).astype(np.float64)
    assert np.all(np.abs(y) == 1.0 / 32)
    c = np.full((1, n), 0.5, dtype=np.float16)
    y = _run(c.view(np.uint16), None, None, n, 1, 1).view(np.float16).astype(np.float64)
    assert y[0, 0] == 16.0 and np.all(y[0, 1:] == 0)
    # twice with no signs and Q = I gives x back (H / sqrt(K) is an involution),
    # up to the two fp16 roundings
    x1, _, _ = _case(n, 1, 1, seed=9, signs=False, q=False)
    y1 = _run(_run(x1, None, None, n, 1, 1), None, None, n, 1, 1)
    a = x1.view(np.float16).astype(np.float64)
    b = y1.view(np.float16).astype(np.float64)
    assert np.all(np.abs(a - b) <= 2 * orot.ulp16(a) + 1e-3)


@pytest.mark.parametrize("rows,n,m,batch,signs,q", [
    (4096, 4096, 1, 1, True, True), (4096, 12288, 3, 1, True, True),
    (4096, 12288, 3, 4, True, True), (1024, 25600, 25, 1, True, True),
    (300, 2560, 5, 2, True, True), (257, 1024 * 19, 19, 1, True, True),
    (64, 256, 1, 3, True, True), (96, 24 * 64, 3, 2, True, True),
    # K from 8 to 64 (lane groups narrower than a wave), every m up to 8, no
    # signs or no Q
    (50, 24, 3, 1, True, True), (64, 48, 6, 2, True, True), (128, 192, 3, 1, True, True),
    (128, 16384, 8, 1, True, True), (200, 2048, 2, 3, True, False),
    (77, 1792, 7, 1, False, True), (64, 4096, 1, 2, False, False), (96, 24 * 64, 3, 2, False, False),
    (40, 4 * 32, 4, 1, True, True),
])
def test_gemv_rotated_equals_rotate_then_gemv(rows, n, m, batch, signs, q):
    import synth as sy
    from oracle import gemv as og
    d = sy.leech_matrix(rows, n, 3, key=(rows, n, m))
    blob = to_dev(lvq.expand(d["coords"], d["scale"], d["tail"], rows, n))
    x, words, qm = _case(n, m, batch, seed=rows + n, signs=signs, q=q)
    wd = None if words is None else to_dev(words)
    qd = None if qm is None else to_dev(qm)
    xr = empty((batch, n), np.uint16)
    lvq.rotate(to_dev(x), n, m, wd, qd, xr, batch)
    y_sep = empty((batch, rows), np.float32)
    lvq.gemv(blob, rows, n, xr, y_sep, batch)
    y_fused = empty((batch, rows), np.float32)
    lvq.gemv_rotated(blob, rows, n, wd, qd, m, to_dev(x), y_fused, batch)
    a, b = to_host(y_fused, np.float32), to_host(y_sep, np.float32)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # and against the oracle: the rotated x as the device rounded it, then f64
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], n)
    y64, bound = og.gemv(w, to_host(xr, np.uint16))
    assert og.check(a, y64, bound) <= 1.0
    # the rotated x itself against the rotation oracle
    y64r, bnd = orot.rotate(x, n, m, words, None if qm is None else qm.astype(np.float64))
    assert orot.rotate_check(to_host(xr, np.uint16), y64r, bnd) <= 1.0
