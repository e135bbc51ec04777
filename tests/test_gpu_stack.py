"""GPU parity on the Qwen3-8B-shaped Leech stack (36 layers x q, k, v, o, gate,
up, down), through the C ABI, against the f64 oracle.

Every matrix is drawn at its full size with the stack's per-layer seeds and
the dependent chain is followed: q, k and v take the layer input, o takes
renorm(q), gate and up take renorm(o), down takes renorm(up), and the next
layer's input is renorm(down), with renorm(v) = fp16((v - mean v) / std v)
in f64.  Each GEMV is checked on exactly the fp16 input it was given.  The
first and the last layer are run (the middle ones differ only in their seeds;
drawing all 36 takes minutes on one core), the last one fed from the first
one's output.
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


def _gemv(d, x_bits):
    rows, cols = d["rows"], d["cols"]
    blob = lvq.expand(d["coords"], d["scale"], d["tail"], rows, cols)
    yd = empty((1, rows), np.float32)
    lvq.gemv(to_dev(blob), rows, cols, to_dev(x_bits), yd, 1)
    y = to_host(yd, np.float32)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], cols)
    y64, bound = og.gemv(w, x_bits)
    r = og.check(y, y64, bound)
    print("layer %d %-4s %5dx%-5d: max |err| / (1e-4 * bound) = %.3g"
          % (d["layer"], d["name"], rows, cols, r), flush=True)
    assert r <= 1.0
    return y[0]


def _layer(layer, h):
    mats = []
    for m in range(len(synth.QWEN3_8B_MATRICES)):
        d = synth.qwen3_8b_matrix(layer, m)
        d["layer"] = layer
        mats.append(d)
    q, k, v, o, gate, up, down = mats
    yq = _gemv(q, h)
    _gemv(k, h)
    _gemv(v, h)
    yo = _gemv(o, synth.renorm_bits(yq)[None, :])
    xg = synth.renorm_bits(yo)[None, :]
    _gemv(gate, xg)
    yu = _gemv(up, xg)
    yd = _gemv(down, synth.renorm_bits(yu)[None, :])
    return synth.renorm_bits(yd)[None, :]


def test_qwen3_8b_stack_first_and_last_layer():
    h = synth.activations(4096, 1, 5, key=(0,))
    h = _layer(0, h)
    h = _layer(synth.QWEN3_8B_LAYERS - 1, h)
    assert h.shape == (1, 4096) and np.all(np.isfinite(h.view(np.float16)))
