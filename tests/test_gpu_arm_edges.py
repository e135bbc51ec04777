"""GPU special cases of the two comparison arms and the dense control, through
the C ABI, against the f64 oracle.

BPDQ (model card "Qwen3-8B - 2-bit BPDQ (packed)", section Format): a weight is
c0 b0 + c1 b1 + c2 per (group of 256 columns, row).  All-zero codes leave
only the offsets, y = sum_g c2 * sum_(c in g) x_c; all-one codes give every
weight c0 + c1 + c2; a one-hot x at column c picks w[r, c] out exactly (the
three fp16 coefficients and 0/1 bits sum exactly in fp32), at the edges of a
16-column code word, of a 64-column quarter and of a 256-column group.

Trellis (blog "Qwen3.8-27B on a 12 GB card", sections "A trellis is a codebook
you walk" and "The codebook is a hash"): a one-hot x at column c gives
s_r * T[state(r, c)] exactly (an fp16 x fp16 product is exact in fp32), at
the first eight columns of a packet, whose states wrap to the packet's end
(tail-biting), and at its last column; rows of all-0 and all-3 symbols have
one state everywhere (0x0000 and 0xFFFF).

fp16 control: batch 4 at 4096 x 4096, the batch the Leech arm is also timed at.
"""
import numpy as np
import pytest

import synth
from oracle import gemv as og

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_gemv_lvq_amd as lvq  # noqa: E402
from gpu_util import empty, to_dev, to_host  # noqa: E402


def _one_hot(cols, where):
    """fp16 bits [len(where)][cols]: batch row b is 1.0 at column where[b]."""
    x = np.zeros((len(where), cols), dtype=np.uint16)
    for b, c in enumerate(where):
        x[b, c] = 0x3C00  # 1.0
    return x


# ---------------------------------------------------------------- BPDQ

def _bpdq(codes, coeffs, rows, cols, x):
    batch = x.shape[0]
    yd = empty((batch, rows), np.float32)
    lvq.bpdq_gemv(to_dev(codes), to_dev(coeffs), rows, cols, to_dev(x), yd, batch)
    return to_host(yd, np.float32)


@pytest.mark.parametrize("fill", [0x00000000, 0xFFFFFFFF])
def test_bpdq_constant_codes(fill):
    rows, cols = 4096, 4096
    d = synth.bpdq_matrix(rows, cols)
    codes = np.full_like(d["codes"], fill)
    for batch in (1, 4):
        x = synth.activations(cols, batch, 2, rows=rows)
        y = _bpdq(codes, d["coeffs"], rows, cols, x)
        w = og.bpdq_weights(codes, d["coeffs"], rows, cols)
        c = og.f16(d["coeffs"]).reshape(cols // 256, 3, rows)
        per_weight = c[:, 2, :] if fill == 0 else c.sum(axis=1)  # [group][row]
        assert np.array_equal(w, np.repeat(per_weight, 256, axis=0).T)
        y64, bound = og.gemv(w, x)
        r = og.check(y, y64, bound)
        print("bpdq codes %#x b%d: ratio %.3g" % (fill, batch, r), flush=True)
        assert r <= 1.0


def test_bpdq_one_hot_columns_exact():
    rows, cols = 4096, 4096
    d = synth.bpdq_matrix(rows, cols)
    w = og.bpdq_weights(d["codes"], d["coeffs"], rows, cols)
    for where in ([0], [15], [16], [255], [256], [0, 15, 256, 4095]):
        y = _bpdq(d["codes"], d["coeffs"], rows, cols, _one_hot(cols, where))
        for b, c in enumerate(where):
            assert np.array_equal(y[b], w[:, c].astype(np.float32)), (where, b)


# ---------------------------------------------------------------- trellis

def _trellis(d, rows, cols, x):
    batch = x.shape[0]
    yd = empty((batch, rows), np.float32)
    lvq.trellis_gemv(to_dev(d["bits"]), to_dev(d["table"]), to_dev(d["scale"]), rows, cols,
                     to_dev(x), yd, batch)
    return to_host(yd, np.float32)


def test_trellis_one_hot_columns_exact():
    rows, cols = 4096, 12288
    d = synth.trellis_matrix(rows, cols)
    states = og.trellis_states(d["bits"], rows, cols)
    table, scale = og.f16(d["table"]), og.f16(d["scale"])
    cols_to_check = list(range(8)) + [255, 256, 263, 511, cols - 1]
    for b0 in range(0, len(cols_to_check), 4):
        where = cols_to_check[b0:b0 + 4]
        x = _one_hot(cols, where)
        if len(where) * cols > 12288:  # the kernel's batch x cols limit
            ys = np.concatenate([_trellis(d, rows, cols, x[i:i + 1]) for i in range(len(where))])
        else:
            ys = _trellis(d, rows, cols, x)
        for b, c in enumerate(where):
            expect = (scale * table[states[:, c]]).astype(np.float32)
            assert np.array_equal(ys[b], expect), c


@pytest.mark.parametrize("sym", [0, 3])
def test_trellis_constant_symbol_rows(sym):
    rows, cols = 64, 3072
    d = synth.trellis_matrix(rows, cols)
    bits = d["bits"].copy()
    bits[::2] = 0xFFFFFFFF if sym == 3 else 0  # every other row constant
    d = dict(d, bits=bits)
    st = og.trellis_states(bits, rows, cols)
    assert np.all(st[::2] == (0xFFFF if sym == 3 else 0))
    for batch in (1, 4):
        x = synth.activations(cols, batch, 4, rows=rows)
        y = _trellis(d, rows, cols, x)
        y64, bound = og.gemv(og.trellis_weights(bits, d["table"], d["scale"], rows, cols), x)
        r = og.check(y, y64, bound)
        print("trellis constant %d b%d: ratio %.3g" % (sym, batch, r), flush=True)
        assert r <= 1.0


# ---------------------------------------------------------------- fp16 control

def test_fp16_batch4_4096():
    rows, cols, batch = 4096, 4096, 4
    wb = synth.dense_matrix(rows, cols)
    x = synth.activations(cols, batch, 2, rows=rows)
    yd = empty((batch, rows), np.float32)
    lvq.fp16_gemv(to_dev(wb), rows, cols, to_dev(x), yd, batch)
    y64, bound = og.gemv(og.fp16_weights(wb, rows, cols), x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    print("fp16 4096x4096 b4: ratio %.3g" % r, flush=True)
    assert r <= 1.0
    one = _one_hot(cols, [0, 7, 8, 4095])
    yd = empty((4, rows), np.float32)
    lvq.fp16_gemv(to_dev(wb), rows, cols, to_dev(one), yd, 4)
    got = to_host(yd, np.float32)
    w = og.fp16_weights(wb, rows, cols)
    for b, c in enumerate([0, 7, 8, 4095]):
        assert np.array_equal(got[b], w[:, c].astype(np.float32))
