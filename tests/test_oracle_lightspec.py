"""Pins for the oracle's two-stage budget planner (LightSpec article): each
check ties it to something other than itself - numpy's masked mean, the
closed form of an EMA under a constant input, exact reproduction of a linear
table, exhaustive search over every prefix-length vector, and the closed form
of the decode throughput for a constant throughput table."""

import itertools

import numpy as np
import pytest

from oracle import lightspec as L
from oracle import schedule as S
from oracle.verify import ST_NONFINITE, ST_ZERO_Z


def _case(g, R, G):
    alpha = g.uniform(0.0, 1.0, (R, G)).astype(np.float32)
    ell = g.integers(0, G + 1, R)
    status = np.zeros(R, np.int32)
    status[g.integers(0, R)] = ST_NONFINITE
    return alpha, ell, status


def test_first_update_is_the_masked_mean():
    g = np.random.default_rng(1)
    alpha, ell, status = _case(g, 40, 7)
    ema, cnt = L.ema_update(alpha, ell, status, 0.3, np.full(7, 0.5), np.zeros(7, np.int64))
    ok = (status & (ST_NONFINITE | ST_ZERO_Z)) == 0
    for j in range(1, 8):
        sel = ok & (ell >= j)
        assert cnt[j - 1] == sel.sum()
        if sel.any():
            assert np.isclose(ema[j - 1], alpha[sel, j - 1].astype(np.float64).mean(), rtol=1e-14, atol=0)
        else:
            assert ema[j - 1] == 0.5               # never observed: the prior stays


def test_constant_input_follows_the_closed_form():
    lam, m, e0 = 0.2, 0.625, 0.9                   # m exact in fp32
    R, G = 5, 3
    alpha = np.full((R, G), m, np.float32)
    ell = np.full(R, G)
    st = np.zeros(R, np.int32)
    ema, cnt = np.full(G, e0), np.ones(G, np.int64)    # already observed once
    for k in range(1, 40):
        ema, cnt = L.ema_update(alpha, ell, st, lam, ema, cnt)
        assert np.allclose(ema, m + (e0 - m) * (1 - lam) ** k, rtol=0, atol=1e-14)
    assert np.all(cnt == 1 + 39 * R)
    same, _ = L.ema_update(alpha * 0 + 0.1, ell, st, 0.0, ema, cnt)     # lam = 0: frozen
    assert np.array_equal(same, ema)


def test_interpolation_reproduces_a_linear_table():
    G = 11
    true = 0.95 - 0.05 * np.arange(G)
    count = np.zeros(G, np.int64)
    count[[1, 4, 5, 9]] = 3
    ema = np.where(count > 0, true, 123.0)         # unobserved entries hold garbage priors
    got = L.planning_confidences(ema, count)
    inner = np.arange(G)[(np.arange(G) > 1) & (np.arange(G) < 9)]
    assert np.allclose(got[inner], true[inner], rtol=0, atol=1e-15)
    assert got[0] == true[1] and got[10] == true[9]   # held constant past the ends
    none = L.planning_confidences(ema, np.zeros(G, np.int64))
    assert np.array_equal(none, ema)                  # nothing observed: the prior
    assert np.all(L.conf_hat(np.array([1.5, -0.2]), np.array([1, 1])) == [1.0, 0.0])


def _brute(c, R, d_cap, sps):
    """Best (tau, B) over every prefix-length vector with lengths <= d_cap[r],
    smallest B among the maximisers of Theta (Theta = 0 with nothing)."""
    a = S.survival(c[None, :])[0]
    q = [S.fixed_point(float(x)) for x in a]
    best = (0.0, R, 0)
    for ell in itertools.product(*[range(int(d) + 1) for d in d_cap]):
        T = sum(sum(q[:l]) for l in ell)
        B = R + sum(ell)
        th = float(np.float64(T * 2.0 ** -32) * np.float64(sps[B - 1])) if sum(ell) else 0.0
        if th > best[0] or (th == best[0] and B < best[1]):
            best = (th, B, T)
    return best


@pytest.mark.parametrize("seed", range(4))
def test_both_stages_match_exhaustive_search(seed):
    g = np.random.default_rng(20 + seed)
    R, G = 3, 3
    ema = g.uniform(0.2, 1.0, G)
    if seed == 3:
        ema[1] = 1.0                               # a tie between positions
    count = np.ones(G, np.int64)
    sps = g.uniform(0.5, 2.0, R * (G + 1)).astype(np.float32)
    cost = g.uniform(0.0, 1.0, G).astype(np.float32)
    d_prev = g.integers(0, G + 1, R)
    res = L.plan(ema, count, d_prev, sps, cost)
    c = res["conf"]
    th1, B1, _ = _brute(c, R, d_prev, sps)
    assert res["theta"] == th1 and res["B"] == B1
    for d in range(1, G + 1):
        th, B, T = _brute(c, R, [d] * R, sps)
        assert R + res["n_best"][d - 1] == B
        phi = (R + T * 2.0 ** -32) / (float(cost[d - 1]) + 1.0 / float(sps[B - 1]))
        assert np.isclose(res["phi"][d - 1], phi, rtol=1e-15, atol=0)
    assert res["phi"][res["d_next"] - 1] == res["phi"].max()
    assert res["d_next"] == 1 + int(np.argmax(res["phi"]))


def test_constant_throughput_closed_form():
    R, G = 4, 6
    c = np.array([0.9, 0.8, 0.75, 0.5, 0.5, 0.25])
    sps = np.full(R * (G + 1), 2.0, np.float32)
    cost = (0.05 * np.arange(1, G + 1)).astype(np.float32)   # linear draft cost
    res = L.plan(c, np.ones(G, np.int64), np.full(R, G), sps, cost)
    a = np.cumprod(c.astype(np.float32), dtype=np.float32).astype(np.float64)
    for d in range(1, G + 1):
        # Theta grows with n at constant SPS, so every request verifies all d
        assert res["n_best"][d - 1] == R * d
        want = R * (1 + a[:d].sum()) / (float(cost[d - 1]) + 0.5)
        assert np.isclose(res["phi"][d - 1], want, rtol=1e-9)
    assert np.array_equal(res["ell"], np.full(R, G))
