"""GPU parity on the whole Qwen3-8B-shaped Leech stack (36 layers x q, k, v,
o, gate, up, down: 252 GEMVs, 4.08 GB of blobs), through the C ABI, against
the f64 oracle.

Every matrix is drawn at its full size with the stack's per-layer seeds and
the dependent chain is followed: q, k and v take the layer input, o takes
renorm(q), gate and up take renorm(o), down takes renorm(up), and the next
layer's input is renorm(down), with renorm(v) = fp16((v - mean v) / std v)
in f64.  Each GEMV is checked on exactly the fp16 input it was given.  The
host work (drawing, expanding, and the oracle's reconstruction for the check)
runs in the worker pool that conftest forks before the GPU runtime starts;
the chain itself runs here, one layer at a time, so device memory holds one
layer's blobs.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_gemv_lvq_amd as lvq  # noqa: E402
import stack_workers  # noqa: E402
from gpu_util import empty, to_dev, to_host  # noqa: E402

_RUN = {}  # the chain's recorded inputs and outputs, shared by the two tests


def test_qwen3_8b_stack_chain(host_pool):
    if host_pool is None:
        pytest.skip("needs the worker pool conftest forks when GPU tests are selected")
    layers = synth.QWEN3_8B_LAYERS
    jobs = [(li, mi) for li in range(layers) for mi in range(len(synth.QWEN3_8B_MATRICES))]
    drawn = host_pool.imap(stack_workers.draw_expand, jobs, chunksize=1)  # in chain order
    records = []
    h = synth.activations(4096, 1, 5, key=(0,))
    for li in range(layers):
        mats = [next(drawn) for _ in range(len(synth.QWEN3_8B_MATRICES))]
        assert [m[:2] for m in mats] == [(li, mi) for mi in range(len(mats))]
        dev = [(rows, cols, to_dev(blob)) for (_, _, rows, cols, blob) in mats]

        def gemv(mi, x_bits):
            rows, cols, bd = dev[mi]
            yd = empty((1, rows), np.float32)
            lvq.gemv(bd, rows, cols, to_dev(x_bits), yd, 1)
            y = to_host(yd, np.float32)
            records.append((li, mi, x_bits, y))
            assert np.all(np.isfinite(y))
            return y[0]

        yq = gemv(0, h)
        gemv(1, h)
        gemv(2, h)
        yo = gemv(3, synth.renorm_bits(yq)[None, :])
        xg = synth.renorm_bits(yo)[None, :]
        gemv(4, xg)
        yu = gemv(5, xg)
        yd_ = gemv(6, synth.renorm_bits(yu)[None, :])
        h = synth.renorm_bits(yd_)[None, :]
        del dev
        torch.cuda.empty_cache()
    assert len(records) == len(jobs)
    _RUN["records"] = records
    print("stack chain: %d GEMVs through %d layers" % (len(records), layers), flush=True)


def test_qwen3_8b_stack_every_gemv_matches_the_oracle(host_pool):
    if "records" not in _RUN:
        pytest.skip("the chain did not run")
    worst = {}
    for li, mi, r, bmin in host_pool.imap_unordered(stack_workers.check, _RUN["records"],
                                                    chunksize=1):
        name = synth.QWEN3_8B_MATRICES[mi][0]
        worst[(li, mi)] = r
        if li in (0, synth.QWEN3_8B_LAYERS - 1) or r > 0.5:
            print("layer %2d %-4s: max |err| / (1e-4 * bound) = %.3g" % (li, name, r), flush=True)
        assert bmin > 0
    assert len(worst) == len(_RUN["records"])
    top = max(worst, key=worst.get)
    print("stack: %d GEMVs checked, worst ratio %.3g (layer %d, %s)"
          % (len(worst), worst[top], top[0], synth.QWEN3_8B_MATRICES[top[1]][0]), flush=True)
    bad = {k: v for k, v in worst.items() if v > 1.0}
    assert not bad, bad
