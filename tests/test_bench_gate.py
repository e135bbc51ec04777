"""The bench's parity gate (bench.OracleLeg), on the CPU: it accepts outputs
within 1e-4 * sum_c |w x| of the f64 oracle, refuses one past it with
ParityGateError (the bench then exits non-zero without a result line), refuses
a failed bit-exact check, and checks nothing when the CPU leg is off.  The
"GPU outputs" here are the oracle's own f64 results rounded to fp32, with one
element moved past the bar."""
import numpy as np
import pytest

import bench
import synth
from oracle import gemv as og


def _leech_case():
    rows, cols, batch = 40, 24 * 6 + 5, 2
    d = synth.leech_matrix(rows, cols, 3)
    d["rows"], d["cols"] = rows, cols
    x = synth.activations(cols, batch, 3, rows=rows)
    y64, bound = og.gemv(og.leech_weights(d["coords"], d["scale"], d["tail"], cols), x)
    return d, x, y64, bound


def test_gate_accepts_the_oracle_and_refuses_past_the_bar():
    d, x, y64, bound = _leech_case()
    leg = bench.OracleLeg(True)
    ok = y64.astype(np.float32)
    r = leg.leech("leech ok", d, x, ok)
    assert r <= 1e-2  # fp32 rounding of the f64 result
    assert leg.ratios["leech ok"] == pytest.approx(r, abs=1e-5)
    bad = ok.copy()
    b, i = np.unravel_index(np.argmax(bound), bound.shape)
    bad[b, i] = y64[b, i] + 1.5e-4 * bound[b, i]  # 1.5x the tolerance
    with pytest.raises(bench.ParityGateError):
        leg.leech("leech bad", d, x, bad)
    assert leg.ratios["leech bad"] > 1.0


def test_gate_refuses_other_arms_and_bit_exact_failures():
    rows, cols = 32, 512
    d = synth.bpdq_matrix(rows, cols)
    x = synth.activations(cols, 1, 2, rows=rows)
    y64, bound = og.gemv(og.bpdq_weights(d["codes"], d["coeffs"], rows, cols), x)
    leg = bench.OracleLeg(True)
    assert leg.bpdq("bpdq ok", d, x, y64.astype(np.float32)) <= 1e-2
    bad = y64.astype(np.float32)
    b, i = np.unravel_index(np.argmax(bound), bound.shape)
    bad[b, i] = y64[b, i] - 2e-4 * bound[b, i]  # 2x the tolerance
    with pytest.raises(bench.ParityGateError):
        leg.bpdq("bpdq bad", d, x, bad)
    assert leg.bitexact("decode ok", True)
    with pytest.raises(bench.ParityGateError):
        leg.bitexact("decode bad", False)


def test_gate_off_checks_nothing():
    d, x, y64, bound = _leech_case()
    leg = bench.OracleLeg(False)
    assert leg.leech("leech", d, x, np.zeros_like(y64, dtype=np.float32) + 1e9) is None
    assert leg.ratios == {}
