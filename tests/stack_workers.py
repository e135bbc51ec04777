"""Host-side work for the Qwen3-8B-shaped stack tests, run in worker processes
(forked before the test process touches the GPU; the workers never use it).

draw_expand: draw one matrix of the stack with its per-layer seeds and expand
it into the Leech blob (the library's host expander).
check: draw the same matrix again and compare a GPU output with the f64
oracle on the exact fp16 input that GPU launch was given.
"""
import numpy as np


def draw_expand(job):
    import dequant_gemv_lvq_amd as lvq
    import synth
    layer, matrix = job
    d = synth.qwen3_8b_matrix(layer, matrix)
    blob = lvq.expand(d["coords"], d["scale"], d["tail"], d["rows"], d["cols"])
    return layer, matrix, d["rows"], d["cols"], blob


def check(job):
    """(layer, matrix, x fp16 bits [1][cols], y fp32 [1][rows]) -> (layer,
    matrix, largest |y - y_f64| / (1e-4 * bound), smallest bound)."""
    import synth
    from oracle import gemv as og
    layer, matrix, x_bits, y = job
    d = synth.qwen3_8b_matrix(layer, matrix)
    w = og.leech_weights(d["coords"], d["scale"], d["tail"], d["cols"])
    y64, bound = og.gemv(w, x_bits)
    return layer, matrix, og.check(np.asarray(y), y64, bound), float(bound.min())
