"""A row's result does not depend on the launch that computes it.

Lane l of a row's wave always takes blocks l, l + 64, l + 128, ... of the row
in column order, into the same accumulators, and the wave reduction is a fixed
tree, so the workgroup size (256 to 1024 threads), the blocks per lane (1 to
4), the waves per row and the number of rows in the launch change no bit of
y.  Here the first k rows of a matrix, expanded as a matrix of their own,
must give the full matrix's first k outputs bit for bit.  With 40 rows the
launch takes 256-thread workgroups and four blocks per lane at 4096x12288
(the full matrix: 1024 threads, two per lane); 2500 rows take 512-thread
workgroups; at batch 3 the blocks per lane are 2 and 1.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_gemv_lvq_amd as lvq  # noqa: E402
from gpu_util import empty, to_dev, to_host  # noqa: E402


def _y(d, k, cols, x, batch, expand, gemv):
    blob = expand(d["coords"][:k], d["scale"][:k], d["tail"][:k], k, cols)
    yd = empty((batch, k), np.float32)
    gemv(to_dev(blob), k, cols, to_dev(x), yd, batch)
    return to_host(yd, np.float32)


@pytest.mark.parametrize("rows,cols", [(4096, 12288), (12288, 4096)])
@pytest.mark.parametrize("batch", [1, 3])
@pytest.mark.parametrize("layout", ["lp3", "direct"])
def test_row_results_do_not_depend_on_the_launch(rows, cols, batch, layout):
    d = synth.leech_matrix(rows, cols, 3)
    x = synth.activations(cols, batch, 3, key=(rows, batch))
    expand, gemv = ((lvq.expand, lvq.gemv) if layout == "lp3" else
                    (lvq.expand_direct, lvq.gemv_direct))
    full = _y(d, rows, cols, x, batch, expand, gemv)
    for k in (40, 2500):
        part = _y(d, k, cols, x, batch, expand, gemv)
        assert np.array_equal(part.view(np.uint32), full[:, :k].view(np.uint32)), (k, layout)
    print("%s %dx%d b%d: first 40 and 2500 rows equal the full launch bit for bit" % (
        layout, rows, cols, batch), flush=True)


def test_each_kernel_keeps_its_own_occupancy():
    """The grid of a launch comes from the occupancy of that kernel: after a
    plain GEMV (two 1024-thread workgroups per CU) has been sized, the fused
    rotation at the same shape (more registers: one workgroup per CU) must
    still get its own, smaller grid.  A cache shared by all kernel variants
    once gave it the plain kernel's grid, half of which then waited for a
    second round (15.5 instead of 11.7 us at 12288 x 4096)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plain = lvq.gemv_launch_info("gemv", 12288, 4096)
    rot = lvq.gemv_launch_info("rotated", 12288, 4096)
    b4 = lvq.gemv_launch_info("gemv", 4096, 12288, batch=4)
    assert plain["threads"] == rot["threads"] == 1024
    assert plain["workgroups"] == 2 * cus
    assert rot["workgroups"] == cus
    assert b4["workgroups"] == cus  # batch 4 at 12288 columns: 96 KiB of x, one per CU
    assert lvq.gemv_launch_info("gemv", 12288, 4096)["workgroups"] == 2 * cus
