"""Pins for the oracle's logical planes and class table."""
import numpy as np

import synth
from oracle import layout, leech


def test_class_table_entries():
    t = layout.class_table()
    assert t.size == 302
    cl = leech.classes()
    for c in cl:
        b = int(t[c["id"]]).to_bytes(8, "little")
        mags = [v for v in b[:5]]
        assert mags[: len(c["mags"])] == list(c["mags"])
        assert all(v == 0 for v in mags[len(c["mags"]):])
        assert b[5] == 0 and b[6] == 0
        assert b[7] & 0x7F == c["m"] and b[7] >> 7 == c["parity"]


def test_planes_roundtrip_and_loop_agree():
    rng = np.random.default_rng(2)
    cl = leech.classes()
    blocks = [np.zeros((1, 24), dtype=np.int8)]
    for c in cl[1:]:
        blocks.append(synth.sample_class(c["key"], 2, rng))
    blocks = np.concatenate(blocks)
    a = layout.expected_planes(blocks)
    b = layout.expected_planes_loop(blocks)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(layout.decode_planes(a), blocks.astype(np.int64))
    # the class id read back from the planes is the class of the point
    for i in range(0, blocks.shape[0], 17):
        assert a["cls"][i] == leech.class_of(blocks[i])


def test_rank_and_sign_meaning():
    x = np.zeros((1, 24), dtype=np.int64)
    x[0, :2] = [4, -4]
    p = layout.expected_planes(x)
    assert p["sign"][0] == 0b10
    # mags (0, 4): rank 1 for the two 4s, rank 0 elsewhere
    assert p["r0"][0] == 0b11 and p["r1"][0] == 0 and p["r2"][0] == 0


def test_byte_counts():
    assert layout.logical_bytes(4096, 12288) == 29368320
    assert layout.logical_bytes(1536, 1536) == 1379328
    assert layout.logical_bytes(4096, 4096) == 9887744
    assert layout.logical_bytes(12288, 4096) == 29663232
    off = layout.sections(4096, 4096)
    assert all(v % 256 == 0 for v in off.values())
    assert off["total"] - layout.logical_bytes(4096, 4096) < 4 * 256 + 302 * 8
