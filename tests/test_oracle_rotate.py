"""Pins of the f64 rotation oracle against things other than itself:
scipy's Hadamard matrix, numpy.kron, H H^T = K I, orthogonality, involution,
and hand-checked special cases."""
import numpy as np
import pytest
import scipy.linalg

import synth
from oracle import rotate as orot
from oracle.gemv import f16


def _x_bits(rng, batch, n, scale=1.0):
    return synth.fp16_bits(rng.standard_normal((batch, n)) * scale)


def _orthogonal(rng, m):
    a, _ = np.linalg.qr(rng.standard_normal((m, m)))
    return a


@pytest.mark.parametrize("k", [1, 2, 4, 8, 64, 1024])
def test_fwht_is_the_sylvester_hadamard_matvec(k):
    rng = np.random.default_rng(k)
    v = rng.standard_normal((3, k))
    want = v @ scipy.linalg.hadamard(k).T.astype(np.float64)
    assert np.allclose(orot.fwht(v), want, rtol=0, atol=1e-12 * np.sqrt(k) * 10)


@pytest.mark.parametrize("k", [1, 2, 16, 256])
def test_fwht_of_identity_gives_h_with_h_ht_equal_k_i(k):
    h = orot.fwht(np.eye(k), axis=0)
    assert np.array_equal(np.abs(h), np.ones((k, k)))
    assert np.array_equal(h @ h.T, k * np.eye(k))
    # Sylvester sign rule (-1)^popcount(a & c)
    a, c = np.meshgrid(np.arange(k), np.arange(k), indexing="ij")
    pop = np.vectorize(lambda t: bin(t).count("1"))(a & c)
    assert np.array_equal(h, np.where(pop % 2 == 1, -1.0, 1.0))


@pytest.mark.parametrize("k,m", [(8, 3), (4, 5), (16, 1), (1, 7), (2, 17)])
def test_rotate_equals_dense_kronecker(k, m):
    rng = np.random.default_rng(100 * k + m)
    n = k * m
    x = _x_bits(rng, 2, n)
    q = _orthogonal(rng, m)
    words = rng.integers(0, 1 << 32, (n + 31) // 32, dtype=np.uint64).astype(np.uint32)
    s = np.array([-1.0 if (int(words[j // 32]) >> (j % 32)) & 1 else 1.0 for j in range(n)])
    dense = np.kron(scipy.linalg.hadamard(k).astype(np.float64), q) / np.sqrt(k)
    want = (f16(x) * s) @ dense.T
    y, bound = orot.rotate(x, n, m, words, q)
    assert np.allclose(y, want, rtol=0, atol=1e-12)
    want_bound = np.abs(f16(x)) @ np.abs(dense).T
    assert np.allclose(bound, want_bound, rtol=1e-12, atol=0)


def test_rotate_is_orthogonal_and_an_involution():
    rng = np.random.default_rng(7)
    n = 4096
    x = _x_bits(rng, 3, n)
    y, _ = orot.rotate(x, n)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(f16(x), axis=1), rtol=1e-13)
    # H / sqrt(K) is symmetric and orthogonal: applying it twice gives x back
    yy = orot.fwht(y, axis=1) / np.sqrt(n)
    assert np.allclose(yy, f16(x), rtol=0, atol=1e-12)
    # with an orthogonal Q and signs the norm is kept too
    q = _orthogonal(rng, 3)
    x3 = _x_bits(rng, 1, 3 * 1024)
    words = rng.integers(0, 1 << 32, 96, dtype=np.uint64).astype(np.uint32)
    y3, _ = orot.rotate(x3, 3 * 1024, 3, words, q)
    assert np.isclose(np.linalg.norm(y3), np.linalg.norm(f16(x3)), rtol=1e-13)


def test_rotate_special_cases():
    # a unit vector e_j (m = 1) maps to column j of H / sqrt(K)
    k = 32
    for j in (0, 5, 31):
        x = np.zeros((1, k), dtype=np.float16)
        x[0, j] = 1.0
        y, _ = orot.rotate(x.view(np.uint16), k)
        col = scipy.linalg.hadamard(k)[:, j] / np.sqrt(k)
        assert np.array_equal(y[0], col)
    # K = 1: y = Q (S x)
    rng = np.random.default_rng(3)
    q = _orthogonal(rng, 5)
    x = _x_bits(rng, 1, 5)
    y, _ = orot.rotate(x, 5, 5, np.array([0b10110], dtype=np.uint32), q)
    s = np.array([1, -1, -1, 1, -1], dtype=np.float64)
    assert np.allclose(y[0], q @ (f16(x)[0] * s), rtol=0, atol=1e-15)
    # every sign bit set negates the result
    x = _x_bits(rng, 1, 64)
    y0, _ = orot.rotate(x, 64)
    y1, _ = orot.rotate(x, 64, 1, np.full(2, 0xFFFFFFFF, dtype=np.uint32))
    assert np.array_equal(y1, -y0)
    # the constant vector concentrates in output 0
    y, _ = orot.rotate(synth.fp16_bits(np.ones((1, 256))), 256)
    assert y[0, 0] == 16.0 and np.all(y[0, 1:] == 0)


def test_rotate_check_bar():
    # a device result that is the fp16 rounding of y64 passes; one off by two
    # ulps fails
    rng = np.random.default_rng(11)
    x = _x_bits(rng, 1, 1024)
    y, bound = orot.rotate(x, 1024)
    rounded = y.astype(np.float16).view(np.uint16)
    assert orot.rotate_check(rounded, y, bound) <= 1.0
    bad = rounded.copy()
    bad[0, 10] += 3
    assert orot.rotate_check(bad, y, bound) > 1.0
    assert orot.ulp16(1.0) == 2.0 ** -10 and orot.ulp16(0.0) == 2.0 ** -24
