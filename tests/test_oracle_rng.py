"""Pins for the oracle's counter-hash uniforms."""

import os

import numpy as np
from scipy import stats

from oracle import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed1234567.txt")


def _golden_values():
    with open(GOLDEN) as f:
        return [int(line) for line in f if line.strip() and not line.startswith("#")]


def test_splitmix64_reference_sequence():
    assert rng.splitmix64_sequence(1234567, 5) == _golden_values()


def test_sm_is_one_generator_step():
    # sm(seed) is the first output of the generator seeded with `seed`.
    for seed in (0, 1, 1234567, 2**64 - 1):
        assert rng.sm(seed) == rng.splitmix64_sequence(seed, 1)[0]


def test_uniform_range_and_resolution():
    u = rng.uniforms(7, np.arange(100000), 3, 1)
    assert u.min() >= 0.0 and u.max() <= 1.0 - 2.0 ** -24
    # every value is a multiple of 2**-24 (24 random bits, fp32-exact)
    assert np.all(np.floor(u * 2 ** 24) == u * 2 ** 24)
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_vectorised_matches_scalar():
    g = np.random.default_rng(5)
    rs = g.integers(0, 5000, 300)
    ps = g.integers(0, 2**40, 300)
    for draw in (0, 1, 2, 3):
        vec = rng.uniforms(0xC0FFEE, rs, ps, draw)
        sca = [rng.uniform(0xC0FFEE, int(r), int(p), draw) for r, p in zip(rs, ps)]
        assert np.array_equal(vec, np.array(sca))


def test_chi_square_uniformity():
    n, bins = 1 << 20, 1 << 12
    r = np.arange(n) % 4096
    pos = np.arange(n) // 4096
    u = rng.uniforms(12345, r, pos, 1)
    counts = np.bincount((u * bins).astype(np.int64), minlength=bins)
    _, pval = stats.chisquare(counts)
    assert pval > 1e-4


def test_draws_are_independent():
    # 2-D chi-square on (accept uniform, correction uniform) of the same counter.
    n = 1 << 18
    r = np.arange(n) % 512
    pos = np.arange(n) // 512
    a = (rng.uniforms(99, r, pos, 1) * 16).astype(np.int64)
    b = (rng.uniforms(99, r, pos, 2) * 16).astype(np.int64)
    table = np.bincount(a * 16 + b, minlength=256).reshape(16, 16)
    _, pval, _, _ = stats.chi2_contingency(table)
    assert pval > 1e-4
