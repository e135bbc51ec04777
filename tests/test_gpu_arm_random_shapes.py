"""GPU parity of the comparison arms and the fp16 control over seeded random
shapes, through the C ABI, against the f64 oracle: rows 1..2100, every width
class each kernel's launch distinguishes (BPDQ: 16, 32 or 64 quarter-group
slots per workgroup row by width; trellis: 256-column packets, 1..48 per
row; fp16: any multiple of 8 columns, so ragged 16-byte units), batch 1..4
within each entry point's batch x cols limit.  Fixed cases cover the
workload shapes and the special values; these sweep the launch choices in
between."""
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

ROWS = [1, 3, 16, 17, 100, 257, 1024, 2100]


def _batch(rng, cols, limit):
    return int(rng.integers(1, min(4, limit // cols) + 1))


def _cases(kind, n=12):
    rng = np.random.default_rng({"bpdq": 71, "trellis": 72, "fp16": 73}[kind])
    out = []
    for i in range(n):
        rows = int(rng.choice(ROWS))
        if kind == "bpdq":
            cols = 256 * int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 17, 24, 32, 40]))
            batch = _batch(rng, cols, 65536)
        elif kind == "trellis":
            cols = 256 * int(rng.choice([1, 2, 3, 5, 8, 12, 16, 24, 48]))
            batch = _batch(rng, cols, 12288)
        else:
            cols = 8 * int(rng.integers(1, 1537))
            batch = _batch(rng, cols, 65536)
        out.append((i, rows, cols, batch))
    return out


def _ids(c):
    return "s%d-%dx%d-b%d" % c


def _report(name, r):
    print("%s: max |y - y64| / (1e-4 sum|w x|) = %.4f" % (name, r), flush=True)


@pytest.mark.parametrize("case", _cases("bpdq"), ids=_ids)
def test_bpdq_random_shapes(case):
    i, rows, cols, batch = case
    d = synth.bpdq_matrix(rows, cols, cfg=200 + i)
    x = synth.activations(cols, batch, 2, key=(i, 31))
    yd = empty((batch, rows), np.float32)
    lvq.bpdq_gemv(to_dev(d["codes"]), to_dev(d["coeffs"]), rows, cols, to_dev(x), yd, batch)
    y64, bound = og.gemv(og.bpdq_weights(d["codes"], d["coeffs"], rows, cols), x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    _report("bpdq %s" % _ids(case), r)
    assert r <= 1.0


@pytest.mark.parametrize("case", _cases("trellis"), ids=_ids)
def test_trellis_random_shapes(case):
    i, rows, cols, batch = case
    d = synth.trellis_matrix(rows, cols, cfg=300 + i)
    x = synth.activations(cols, batch, 4, key=(i, 37))
    yd = empty((batch, rows), np.float32)
    lvq.trellis_gemv(to_dev(d["bits"]), to_dev(d["table"]), to_dev(d["scale"]), rows, cols,
                     to_dev(x), yd, batch)
    y64, bound = og.gemv(og.trellis_weights(d["bits"], d["table"], d["scale"], rows, cols), x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    _report("trellis %s" % _ids(case), r)
    assert r <= 1.0


@pytest.mark.parametrize("case", _cases("fp16"), ids=_ids)
def test_fp16_random_shapes(case):
    i, rows, cols, batch = case
    wb = synth.dense_matrix(rows, cols, cfg=400 + i)
    x = synth.activations(cols, batch, 2, key=(i, 41))
    yd = empty((batch, rows), np.float32)
    lvq.fp16_gemv(to_dev(wb), rows, cols, to_dev(x), yd, batch)
    y64, bound = og.gemv(og.fp16_weights(wb, rows, cols), x)
    r = og.check(to_host(yd, np.float32), y64, bound)
    _report("fp16 %s" % _ids(case), r)
    assert r <= 1.0


# ---------------------------------------------------------------- the largest widths

@pytest.mark.parametrize("kind,rows,cols,batch", [
    ("bpdq", 16, 63488, 1),   # the widest that fits LDS at batch 1
    ("bpdq", 16, 32768, 2), ("bpdq", 17, 21760, 3), ("bpdq", 32, 16384, 4),  # batch x cols
    ("trellis", 16, 6144, 2), ("trellis", 3, 12288, 1),
    ("fp16", 16, 65536, 1), ("fp16", 5, 16384, 4),
])
def test_arms_at_their_largest_widths(kind, rows, cols, batch):
    case = (99, rows, cols, batch)
    {"bpdq": test_bpdq_random_shapes, "trellis": test_trellis_random_shapes,
     "fp16": test_fp16_random_shapes}[kind](case)


def test_bpdq_past_the_lds_is_refused():
    # 63,744 columns at batch 1 pass the batch x cols bound but not the LDS
    rows, cols = 16, 63744
    d = synth.bpdq_matrix(rows, cols)
    x = synth.activations(cols, 1, 2)
    yd = empty((1, rows), np.float32)
    with pytest.raises(lvq.LvqError) as e:
        lvq.bpdq_gemv(to_dev(d["codes"]), to_dev(d["coeffs"]), rows, cols, to_dev(x), yd, 1)
    assert e.value.code == lvq.LVQ_E_SHAPE
