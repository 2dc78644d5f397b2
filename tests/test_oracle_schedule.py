"""Pins for the oracle's prefix scheduler.

Each check ties the oracle to something other than itself: numpy's cumulative
product, an exhaustive search over every prefix-length vector, an independent
frontier greedy that recomputes tau from scratch, closed-form special cases,
and the Figure 1 construction of the DSpark summary page.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import schedule as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(g, R, gmax, ragged=True, levels=None):
    if levels is None:
        conf = (1.0 / (1.0 + np.exp(-g.normal(1.0, 1.5, (R, gmax))))).astype(np.float32)
    else:  # few distinct values -> many exact survival ties
        conf = g.choice(np.array(levels, np.float32), size=(R, gmax))
    gam = g.integers(1, gmax + 1, R) if ragged else np.full(R, gmax)
    sps = g.uniform(0.2, 2.0, R * (1 + gmax)).astype(np.float32)
    return conf, gam, sps


def _theta_of(ell, conf, gam, sps):
    """Theta for an arbitrary prefix-length vector, tau summed per request."""
    R = len(ell)
    total = 0
    for r in range(R):
        prod = np.float32(1.0)
        for j in range(int(ell[r])):
            prod = np.float32(prod * conf[r, j])
            total += int(np.rint(np.float64(prod) * 2.0 ** 32))
    B = R + int(sum(ell))
    return float(np.float64(total * 2.0 ** -32) * np.float64(sps[B - 1]))


def test_survival_matches_numpy_cumprod():
    g = np.random.default_rng(1)
    conf = g.uniform(0.01, 1.0, (64, 16)).astype(np.float32)
    a = S.survival(conf)
    ref = np.cumprod(conf, axis=1, dtype=np.float32)
    assert np.array_equal(a, ref)


def test_survival_ragged_zero_tail():
    conf = np.full((2, 4), 0.5, np.float32)
    a = S.survival(conf, [2, 4])
    assert np.array_equal(a[0], np.array([0.5, 0.25, 0, 0], np.float32))
    assert np.array_equal(a[1], np.array([0.5, 0.25, 0.125, 0.0625], np.float32))


def test_fixed_point_exact():
    assert S.fixed_point(1.0) == 2 ** 32
    assert S.fixed_point(0.5) == 2 ** 31
    assert S.fixed_point(2.0 ** -33) == 0          # tie at 0.5 rounds to even 0
    assert S.fixed_point(3 * 2.0 ** -33) == 2      # tie at 1.5 rounds to even 2
    assert S.fixed_point(float(np.float32(2.0 ** -20 * 1.5))) == 3 * 2 ** 11


@pytest.mark.parametrize("levels", [None, [0.25, 0.5, 0.75, 1.0]])
def test_global_argmax_equals_exhaustive_max(levels):
    g = np.random.default_rng(2 if levels is None else 3)
    for _ in range(400):
        R = int(g.integers(1, 5))
        gmax = int(g.integers(1, 5))
        conf, gam, sps = _rand_case(g, R, gmax, levels=levels)
        res = S.schedule(conf, sps, S.GLOBAL_ARGMAX, gam)
        best = max(_theta_of(ell, conf, gam, sps)
                   for ell in itertools.product(*[range(int(x) + 1) for x in gam]))
        assert res["theta"] == best
        assert _theta_of(res["ell"], conf, gam, sps) == best
        early = S.schedule(conf, sps, S.EARLY_STOP, gam)
        assert early["theta"] <= best


def _frontier_greedy(conf, gam, sps):
    """Independent early-stop greedy: pick the best next draft per request."""
    R = conf.shape[0]
    ell = [0] * R
    theta_prev = 0.0
    while True:
        best_r, best_a = None, None
        for r in range(R):
            if ell[r] < gam[r]:
                a = np.float32(1.0)
                for j in range(ell[r] + 1):
                    a = np.float32(a * conf[r, j])
                if best_a is None or a > best_a:
                    best_r, best_a = r, a
        if best_r is None:
            return ell
        trial = list(ell)
        trial[best_r] += 1
        th = _theta_of(trial, conf, gam, sps)
        if th < theta_prev:
            return ell
        ell, theta_prev = trial, th


@pytest.mark.parametrize("levels", [None, [0.5, 1.0]])
def test_early_stop_equals_frontier_greedy(levels):
    g = np.random.default_rng(4 if levels is None else 5)
    for _ in range(1500):
        R = int(g.integers(1, 5))
        gmax = int(g.integers(1, 5))
        conf, gam, sps = _rand_case(g, R, gmax, levels=levels)
        res = S.schedule(conf, sps, S.EARLY_STOP, gam)
        assert list(res["ell"]) == _frontier_greedy(conf, gam, sps)
        assert res["B"] == R + int(res["ell"].sum())


def test_constant_sps_takes_everything():
    g = np.random.default_rng(6)
    conf, gam, _ = _rand_case(g, 8, 6)
    sps = np.full(8 * 7, 3.0, np.float32)
    res = S.schedule(conf, sps, S.EARLY_STOP, gam)
    assert np.array_equal(res["ell"], gam.astype(np.int32))


def test_early_stop_matches_argmax_when_unimodal():
    # A throughput table that rises then falls keeps Theta unimodal.
    g = np.random.default_rng(7)
    for _ in range(200):
        R, gmax = 4, 4
        conf, gam, _ = _rand_case(g, R, gmax, ragged=False)
        B = np.arange(1, R * (1 + gmax) + 1, dtype=np.float64)
        sps = (100.0 / (1.0 + 0.3 * B)).astype(np.float32)  # steps/s falling with B
        e = S.schedule(conf, sps, S.EARLY_STOP)
        a = S.schedule(conf, sps, S.GLOBAL_ARGMAX)
        th = a["thetas"]
        peak = int(np.argmax(th))
        if all(th[i] <= th[i + 1] for i in range(peak)) and all(
                th[i] >= th[i + 1] for i in range(peak, len(th) - 1)):
            assert e["theta"] == a["theta"]


def test_sawtooth_early_stop_is_local():
    # A sawtooth table makes the naive early stop halt at a local optimum
    # ("challenge 2" of the DSpark summary notes real curves are non-monotone).
    R, gmax = 8, 8
    conf = np.full((R, gmax), np.float32(0.95))
    Bs = np.arange(1, R * (1 + gmax) + 1)
    saw = ((Bs - 1) % 8) / 4.0 - 1.0
    sps = (Bs / (1 + Bs / 64.0) * (1 + 0.2 * saw)).astype(np.float32)
    e = S.schedule(conf, sps, S.EARLY_STOP)
    a = S.schedule(conf, sps, S.GLOBAL_ARGMAX)
    assert e["theta"] < a["theta"]
    assert e["B"] < a["B"]


def test_ties_by_request_then_position():
    conf = np.full((3, 2), np.float32(0.5))
    sps = np.ones(9, np.float32)
    res = S.schedule(conf, sps, S.CAPPED_TOPK, cap_k=2)
    # survivals: 0.5, 0.25 for every request -> first the three 0.5s by r
    assert list(res["ell"]) == [1, 1, 0]
    order = [(r, j) for (_a, r, j) in res["order"]]
    assert order == [(0, 1), (1, 1), (2, 1), (0, 2), (1, 2), (2, 2)]


def test_capped_topk_exact_and_clamped():
    g = np.random.default_rng(8)
    conf, gam, sps = _rand_case(g, 6, 5)
    N = int(gam.sum())
    for K in (0, 1, 3, N, N + 10):
        res = S.schedule(conf, sps, S.CAPPED_TOPK, gam, cap_k=K)
        assert res["n_sel"] == min(K, N)
        assert int(res["ell"].sum()) == min(K, N)


def test_async_capacity_from_previous_step():
    g = np.random.default_rng(9)
    conf, gam, sps = _rand_case(g, 6, 5)
    prev, _, _ = _rand_case(g, 6, 5)
    res = S.async_schedule(conf, prev, sps, gam)
    k = S.schedule(prev, sps, S.GLOBAL_ARGMAX, gam)["n_sel"]
    assert res["cap_k"] == k
    assert int(res["ell"].sum()) == k
    # selected set = top-k of the current survivals (prefix-closed per request)
    top = res["order"][:k]
    for r in range(6):
        js = sorted(j for (_a, rr, j) in top if rr == r)
        assert js == list(range(1, len(js) + 1))


def test_figure1_construction():
    with open(os.path.join(GOLDEN, "fig1_schedule.json")) as f:
        case = json.load(f)
    conf = np.array([case["conf"]], np.float32)
    sps = np.array(case["sps"], np.float32)
    res = S.schedule(conf, sps, S.EARLY_STOP)
    assert list(res["ell"]) == case["expected_ell"]
    assert res["B"] == case["expected_B"]


# --- sequential temperature scaling and the threshold mode -------------------

def test_sts_matches_expit_of_scaled_logit():
    from scipy.special import expit, logit
    g = np.random.default_rng(11)
    conf = g.uniform(0.001, 0.999, (6, 7)).astype(np.float32)
    temps = g.uniform(0.3, 3.0, 7)
    got = S.sts(conf, temps).astype(np.float64)
    want = expit(logit(conf.astype(np.float64)) / temps[None, :])
    assert np.allclose(got, want, rtol=2 ** -23, atol=0)


def test_sts_identity_symmetry_and_limits():
    g = np.random.default_rng(12)
    conf = g.uniform(0.0, 1.0, (5, 4)).astype(np.float32)
    conf[0, 0], conf[0, 1], conf[1, 0] = 0.0, 1.0, 0.5
    assert np.array_equal(S.sts(conf, np.ones(4)), conf)           # T = 1: unchanged, bit for bit
    t = np.array([0.5, 2.0, 7.0, 0.25])
    out = S.sts(conf, t)
    assert out[0, 0] == 0.0 and out[0, 1] == 1.0 and out[1, 0] == 0.5
    mirrored = S.sts((1.0 - conf.astype(np.float64)).astype(np.float32), t)
    inner = (conf > 0) & (conf < 1) & (np.abs(1.0 - conf.astype(np.float64) - (1.0 - conf)) == 0)
    assert np.allclose(mirrored[inner], 1.0 - out[inner], atol=1e-7)   # sigma(-z) = 1 - sigma(z)
    big = S.sts(conf, np.full(4, 1e6))
    inner = (conf > 0) & (conf < 1)
    assert np.allclose(big[inner], 0.5, atol=1e-5)                       # T -> inf: 1/2
    # a temperature above 1 pulls every confidence toward 1/2, below 1 away from it
    hot, cold = S.sts(conf, np.full(4, 2.0)), S.sts(conf, np.full(4, 0.5))
    d = np.abs(conf - 0.5)
    assert np.all(np.abs(hot - 0.5)[inner] <= d[inner] + 1e-7)
    assert np.all(np.abs(cold - 0.5)[inner] >= d[inner] - 1e-7)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_threshold_mode_is_the_per_request_definition(seed):
    g = np.random.default_rng(100 + seed)
    conf, gam, sps = _rand_case(g, 9, 6, ragged=True, levels=[0.3, 0.6, 0.9, 1.0] if seed == 2 else None)
    a = S.survival(conf, gam)
    for theta in (0.0, 0.05, 0.3, float(a[0, 0]), 0.81, 1.0, 1.5):
        res = S.schedule(conf, sps, S.THRESHOLD, gam, threshold=theta)
        for r in range(9):
            js = [j for j in range(1, gam[r] + 1) if a[r, j - 1] >= np.float32(theta)]
            assert res["ell"][r] == (max(js) if js else 0)
            assert js == list(range(1, len(js) + 1))                     # a prefix of the draft
        assert res["B"] == 9 + int(res["ell"].sum())


def test_sts_applies_before_the_survival_products():
    g = np.random.default_rng(13)
    conf, gam, sps = _rand_case(g, 5, 5)
    temps = g.uniform(0.5, 2.0, 5)
    res = S.schedule(conf, sps, S.GLOBAL_ARGMAX, gam, sts_temp=temps)
    assert np.array_equal(res["surv"], S.survival(S.sts(conf, temps), gam))
    plain = S.schedule(S.sts(conf, temps), sps, S.GLOBAL_ARGMAX, gam)
    assert np.array_equal(res["ell"], plain["ell"]) and res["theta"] == plain["theta"]
