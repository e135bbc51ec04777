"""Pins for the oracle's f64 reconstruction and matvec, arm by arm.

Each arm is checked against something other than its own formula: exact
rational arithmetic on tiny shapes, special inputs whose result is fixed by
the definition (one-hot and all-ones activations, zero scale, zero blocks),
the pages' worked trellis example, and the BPDQ peel order of the model card.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import gemv, leech

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fr16(bits):
    return Fraction(float(np.uint16(bits).view(np.float16)))


def _exact_y(w_fr, x_fr):
    return [sum((wr[c] * x_fr[c] for c in range(len(x_fr))), Fraction(0)) for wr in w_fr]


# ------------------------------------------------------------------ Leech

def test_leech_matches_exact_rational_tiny():
    d = synth.leech_matrix(3, 50, 3, key=(99,))
    x = synth.activations(50, 1, 3, key=(99,))
    w = gemv.leech_weights(d["coords"], d["scale"], d["tail"], 50)
    y, bound = gemv.gemv(w, x)
    # exact: s_r * coords for 48 block columns, tail values for the last 2
    for r in range(3):
        s = _fr16(d["scale"][r])
        row = [s * int(v) for v in d["coords"][r].reshape(-1)]
        row += [_fr16(t) for t in d["tail"][r]]
        xs = [_fr16(v) for v in x[0]]
        exact = sum((a * b for a, b in zip(row, xs)), Fraction(0))
        babs = sum((abs(a * b) for a, b in zip(row, xs)), Fraction(0))
        assert abs(Fraction(y[0, r]) - exact) <= Fraction(1, 10 ** 12) * babs
        assert abs(Fraction(bound[0, r]) - babs) <= Fraction(1, 10 ** 12) * babs


def test_leech_tail_is_unscaled_and_last():
    d = synth.leech_matrix(2, 30, 3, key=(7,))
    w = gemv.leech_weights(d["coords"], d["scale"], d["tail"], 30)
    assert np.array_equal(w[:, 24:], gemv.f16(d["tail"]))
    s = gemv.f16(d["scale"])
    assert np.array_equal(w[:, :24], d["coords"].reshape(2, 24) * s[:, None])


def test_leech_special_activations():
    rows, cols = 4, 72
    d = synth.leech_matrix(rows, cols, 3, key=(5,))
    d["scale"][1] = 0  # zero scale: the row reads only its (empty) tail
    d["coords"][2, 1] = 0  # one zero block
    w = gemv.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    s = gemv.f16(d["scale"])
    for c in (0, 25, 71):
        x = np.zeros((1, cols), dtype=np.float16)
        x[0, c] = 1
        y, _ = gemv.gemv(w, x.view(np.uint16))
        k, j = divmod(c, 24)
        assert np.array_equal(y[0], s * d["coords"][:, k, j])
    ones = np.ones((1, cols), dtype=np.float16).view(np.uint16)
    y, _ = gemv.gemv(w, ones)
    assert np.array_equal(y[0], s * d["coords"].reshape(rows, -1).sum(axis=1))
    assert y[0, 1] == 0


def test_parity_ratio_semantics():
    y64 = np.array([[1.0, 0.0, -2.0]])
    bound = np.array([[10.0, 0.0, 4.0]])
    assert gemv.check(np.array([[1.0 + 9e-4, 0.0, -2.0]]), y64, bound) < 1
    assert gemv.check(np.array([[1.0 + 2e-3, 0.0, -2.0]]), y64, bound) > 1
    assert gemv.check(np.array([[1.0, 1e-30, -2.0]]), y64, bound) == np.inf
    assert gemv.check(np.array([[1.0, -0.0, -2.0]]), y64, bound) == 0


def test_bound_is_sum_of_abs_products():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((5, 40))
    x = synth.fp16_bits(rng.standard_normal((2, 40)))
    y, b = gemv.gemv(w, x)
    xf = gemv.f16(x)
    for bb in range(2):
        for r in range(5):
            assert np.isclose(b[bb, r], np.sum(np.abs(w[r] * xf[bb])), rtol=1e-13)
            assert np.isclose(y[bb, r], np.sum(w[r] * xf[bb]), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ BPDQ

def _bpdq_peel(codes, coeffs_bits, rows, cols):
    """Model card order: per word, code = word & 3; word >>= 2, 16 times."""
    fmt = json.load(open(os.path.join(GOLDEN, "bpdq_format.json")))
    g = fmt["group_size"]
    coeffs = gemv.f16(coeffs_bits).reshape(cols // g, 3, rows)
    w = np.zeros((rows, cols))
    for i in range(cols // fmt["columns_per_word"]):
        for r in range(rows):
            word = int(codes[i, r])
            for t in range(fmt["columns_per_word"]):
                code = word & 3
                word >>= 2
                c = 16 * i + t
                grp = c // g
                w[r, c] = (coeffs[grp, 0, r] * (code & 1) + coeffs[grp, 1, r] * (code >> 1)
                           + coeffs[grp, 2, r])
    return w


def test_bpdq_matches_peel_order():
    d = synth.bpdq_matrix(8, 512, cfg=2)
    w = gemv.bpdq_weights(d["codes"], d["coeffs"], 8, 512)
    assert np.array_equal(w, _bpdq_peel(d["codes"], d["coeffs"], 8, 512))


def test_bpdq_special_cases():
    rows, cols = 6, 512
    d = synth.bpdq_matrix(rows, cols, cfg=2)
    coeffs = gemv.f16(d["coeffs"]).reshape(2, 3, rows)
    zero = np.zeros_like(d["codes"])
    x = synth.activations(cols, 1, 2, rows=rows)
    y, _ = gemv.gemv(gemv.bpdq_weights(zero, d["coeffs"], rows, cols), x)
    xf = gemv.f16(x)[0]
    expect = coeffs[0, 2] * xf[:256].sum() + coeffs[1, 2] * xf[256:].sum()
    assert np.allclose(y[0], expect, rtol=1e-13, atol=0)
    w = gemv.bpdq_weights(d["codes"], d["coeffs"], rows, cols)
    for c in (0, 17, 300):
        onehot = np.zeros((1, cols), dtype=np.float16)
        onehot[0, c] = 1
        y, _ = gemv.gemv(w, onehot.view(np.uint16))
        code = (d["codes"][c // 16] >> np.uint32(2 * (c % 16))) & 3
        g = c // 256
        assert np.array_equal(y[0], coeffs[g, 0] * (code & 1) + coeffs[g, 1] * (code >> 1)
                              + coeffs[g, 2])


# ------------------------------------------------------------------ trellis

def test_trellis_worked_example_from_pages():
    ex = json.load(open(os.path.join(GOLDEN, "trellis_state_example.json")))
    assert gemv.shift_state(ex["entry"], ex["symbol"], ex["T_bits"], ex["L_bits"]) == ex["state"]


def test_trellis_symbol_order_msb_first():
    bits = np.zeros((1, 16), dtype=np.uint32)
    bits[0, 0] = 0xC0000000  # symbol 0 = 3, everything else 0
    sym = gemv.trellis_symbols(bits, 1, 256)
    assert sym[0, 0] == 3 and sym[0, 1:].sum() == 0
    st = gemv.trellis_states(bits, 1, 256)
    # symbol 0 is the newest bits of state 0 and moves up 2 bits per step
    for k in range(8):
        assert st[0, k] == 3 << (2 * k)
    assert st[0, 8] == 0
    bits[0, 0] = 0
    bits[0, 15] = 0x3  # the packet's last symbol wraps into the first 7 states
    st = gemv.trellis_states(bits, 1, 256)
    for k in range(7):
        assert st[0, k] == 3 << (2 * (k + 1))
    assert st[0, 255] == 3


def test_trellis_window_equals_register_walk():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, size=(3, 32), dtype=np.uint64).astype(np.uint32)
    sym = gemv.trellis_symbols(bits, 3, 512)
    st = gemv.trellis_states(bits, 3, 512)
    for r in range(3):
        for p in range(2):
            walk = gemv.trellis_states_walk(sym[r, 256 * p: 256 * (p + 1)])
            assert list(st[r, 256 * p: 256 * (p + 1)]) == walk


def test_trellis_table_and_onehot():
    d = synth.trellis_matrix(4, 512, cfg=4)
    t = gemv.f16(d["table"])
    assert t.size == 65536 and abs(t.mean()) < 0.02 and abs(t.std() - 1) < 0.02
    w = gemv.trellis_weights(d["bits"], d["table"], d["scale"], 4, 512)
    st = gemv.trellis_states(d["bits"], 4, 512)
    s = gemv.f16(d["scale"])
    for c in (0, 6, 7, 255, 256, 511):
        x = np.zeros((1, 512), dtype=np.float16)
        x[0, c] = 1
        y, _ = gemv.gemv(w, x.view(np.uint16))
        assert np.array_equal(y[0], s * t[st[:, c]])


# ------------------------------------------------------------------ fp16 control

def test_fp16_dense():
    wb = synth.dense_matrix(3, 40, cfg=2)
    w = gemv.fp16_weights(wb, 3, 40)
    assert np.array_equal(w, wb.view(np.float16).astype(np.float64))
