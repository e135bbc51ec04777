"""The seeded generators draw what their recipes say (checked with the oracle)."""
import numpy as np
from scipy import stats

import synth
from oracle import leech


def test_samples_are_lattice_points_of_their_shell():
    rng = np.random.default_rng(4)
    for m in range(2, 13):
        x = synth.sample_shells(np.full(300, m), rng)
        assert leech.is_leech_batch(x).all()
        assert np.all((x.astype(np.int64) ** 2).sum(axis=1) == 16 * m)


def test_every_class_sampled_is_that_class():
    rng = np.random.default_rng(5)
    for c in leech.classes()[1:]:
        x = synth.sample_class(c["key"], 20, rng)
        assert leech.is_leech_batch(x).all()
        assert {leech.class_of(v) for v in x} == {c["id"]}


def _chi2_p(observed, expected):
    keep = expected > 5
    o = np.append(observed[keep], observed[~keep].sum())
    e = np.append(expected[keep], expected[~keep].sum())
    if e[-1] == 0:
        o, e = o[:-1], e[:-1]
    return stats.chisquare(o, e * o.sum() / e.sum()).pvalue


def test_class_frequencies_uniform_in_shell():
    rng = np.random.default_rng(6)
    for m in (2, 3, 5):
        cl = [c for c in leech.classes() if c["m"] == m]
        x = synth.sample_shells(np.full(20000, m), rng)
        ids = np.array([leech.class_of(v) for v in x])
        obs = np.array([(ids == c["id"]).sum() for c in cl], dtype=float)
        exp = np.array([c["count"] for c in cl], dtype=float)
        assert _chi2_p(obs, exp / exp.sum() * obs.sum()) > 1e-4


def test_positions_uniform_within_class():
    # a uniform point of a class puts its largest magnitude on every
    # coordinate equally often
    rng = np.random.default_rng(7)
    key = (4, 4) + (0,) * 22
    x = synth.sample_class(key, 24000, rng)
    obs = (np.abs(x) == 4).sum(axis=0).astype(float)
    assert obs.sum() == 2 * 24000
    assert _chi2_p(obs, np.full(24, obs.sum() / 24)) > 1e-4
    signs = np.sign(x[x != 0])
    assert abs(signs.mean()) < 0.03


def test_workload_recipes():
    d = synth.leech_matrix(512, 1536, 1)
    coords = d["coords"].reshape(-1, 24).astype(np.int64)
    zero = (coords == 0).all(axis=1)
    assert abs(zero.mean() - 0.02) < 0.01
    shells = (coords[~zero] ** 2).sum(axis=1) // 16
    assert set(np.unique(shells)) == {2, 3}
    assert abs((shells == 2).mean() - 0.5) < 0.03
    d3 = synth.leech_matrix(256, 4096, 3)
    c3 = d3["coords"].reshape(-1, 24).astype(np.int64)
    sh = (c3 ** 2).sum(axis=1) // 16
    p = 2.0 ** -np.arange(2, 7)
    p /= p.sum()
    obs = np.array([(sh == m).sum() for m in range(2, 7)], dtype=float)
    assert _chi2_p(obs, p * obs.sum()) > 1e-4
    assert d3["tail"].shape == (256, 16)
    s = d3["scale"].view(np.float16).astype(np.float64)
    assert (s >= 0).all() and abs(s.mean() - 0.02 * np.sqrt(2 / np.pi)) < 0.002


def test_seeds_are_stable_and_independent_of_batch():
    a = synth.leech_matrix(8, 96, 3)
    b = synth.leech_matrix(8, 96, 3)
    assert np.array_equal(a["coords"], b["coords"])
    x1 = synth.activations(96, 1, 3)
    x4 = synth.activations(96, 4, 3)
    assert np.array_equal(x1[0], x4[0])
