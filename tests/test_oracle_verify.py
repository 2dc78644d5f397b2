"""Pins for the oracle's rejection-sampling verification.

The pages fix what the result must satisfy rather than how to compute it:
the emitted tokens follow the target law exactly (losslessness), a draft is
accepted with probability min(1, p/q) so the per-position acceptance rate is
sum_x min(p, q) = 1 - TV(p, q) (the confidence label of the DSpark summary,
"2.1"), and with independent positions the mean accepted length is
sum_j prod_{i<=j} alpha_i.  Monte-Carlo tests use fixed seeds and 5-sigma /
1e-4-level bounds.
"""

import numpy as np
import pytest
from scipy import stats

from oracle import verify as Vf
from oracle import rng


def _logits(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64))


def _run_trials(P, Q, n, seed=11, ell=None, tok_seed=0):
    """n independent requests sharing target rows P[0..L] and draft rows Q[0..L-1];
    draft tokens are drawn from Q with numpy (an input, not the method)."""
    L = len(Q) if ell is None else ell
    V = len(P[0])
    tgt = np.stack([_logits(p) for p in P])
    drf = np.stack([_logits(q) for q in Q]) if len(Q) else np.zeros((1, V))
    g = np.random.default_rng(tok_seed)
    gmax = max(len(Q), 1)
    toks = np.zeros((n, gmax), np.int32)
    for j in range(len(Q)):
        toks[:, j] = g.choice(V, size=n, p=Q[j])
    out = Vf.verify(tgt, np.zeros(n, np.int64), drf, np.zeros(n, np.int64), toks,
                    np.full(n, L), V, 1.0, seed)
    return out, toks


def _dirichlet(g, V, conc=1.0):
    return g.dirichlet(np.full(V, conc))


def test_softmax_and_stats_against_scipy():
    from scipy.special import softmax, logsumexp
    g = np.random.default_rng(0)
    x = g.normal(0, 3, 1000)
    for T in (1.0, 0.7, 2.5):
        p, m, Z, s = Vf.row_softmax(x, 1000, T)
        assert s == 0
        assert np.allclose(p, softmax(x / T), rtol=1e-13, atol=0)
        assert np.isclose(m + np.log(Z), logsumexp(x / T), rtol=1e-13)


def test_inverse_cdf_special_cases():
    w = np.array([0.0, 2.0, 0.0, 1.0, 1.0])
    assert Vf.inverse_cdf(w, 0.0)[0] == 1           # first token with mass
    assert Vf.inverse_cdf(w, 0.49)[0] == 1
    assert Vf.inverse_cdf(w, 0.5)[0] == 3           # boundary goes right
    assert Vf.inverse_cdf(w, 1.0 - 2 ** -24)[0] == 4
    assert Vf.inverse_cdf(np.array([0, 0, 5.0, 0]), 0.99)[0] == 2


def test_inverse_cdf_frequencies():
    g = np.random.default_rng(1)
    w = g.uniform(0, 1, 12) * (g.uniform(0, 1, 12) > 0.3)
    n = 60000
    us = rng.uniforms(3, np.arange(n), 0, 0)
    toks = np.array([Vf.inverse_cdf(w, u)[0] for u in us])
    counts = np.bincount(toks, minlength=12)
    assert np.all(counts[w == 0] == 0)
    exp = n * w / w.sum()
    _, pval = stats.chisquare(counts[w > 0], exp[w > 0])
    assert pval > 1e-4


@pytest.mark.parametrize("V,seed", [(8, 1), (16, 2)])
def test_losslessness_first_token(V, seed):
    g = np.random.default_rng(seed)
    P = [_dirichlet(g, V) for _ in range(4)]
    Q = [_dirichlet(g, V) for _ in range(3)]
    n = 40000
    out, _ = _run_trials(P, Q, n, seed=seed)
    first = out["tokens"][:, 0]
    counts = np.bincount(first, minlength=V)
    _, pval = stats.chisquare(counts, n * P[0])
    assert pval > 1e-4


def test_losslessness_second_position():
    # positions are independent here, so the token emitted at position 2
    # (accepted draft or correction) must follow P[1] whenever it exists.
    V = 10
    g = np.random.default_rng(3)
    P = [_dirichlet(g, V, 2.0) for _ in range(4)]
    Q = [_dirichlet(g, V, 2.0) for _ in range(3)]
    n = 40000
    out, _ = _run_trials(P, Q, n, seed=4)
    has2 = out["n_acc"] >= 1
    second = out["tokens"][has2, 1]
    counts = np.bincount(second, minlength=V)
    _, pval = stats.chisquare(counts, has2.sum() * P[1])
    assert pval > 1e-4


def test_accept_rate_is_one_minus_tv():
    V = 12
    g = np.random.default_rng(5)
    P = [_dirichlet(g, V), _dirichlet(g, V)]
    Q = [_dirichlet(g, V)]
    n = 40000
    out, _ = _run_trials(P, Q, n, seed=6)
    alpha = np.minimum(P[0], Q[0]).sum()
    assert np.isclose(alpha, 1.0 - 0.5 * np.abs(P[0] - Q[0]).sum())
    rate = (out["n_acc"] >= 1).mean()
    assert abs(rate - alpha) < 5 * np.sqrt(alpha * (1 - alpha) / n)
    assert np.allclose(out["alpha"][:, 0], alpha, rtol=1e-12)


def test_mean_accepted_length_closed_form():
    V = 8
    g = np.random.default_rng(7)
    P = [_dirichlet(g, V, 3.0) for _ in range(5)]
    Q = [0.5 * P[j] + 0.5 * _dirichlet(g, V, 3.0) for j in range(4)]
    alphas = [np.minimum(P[j], Q[j]).sum() for j in range(4)]
    expect = sum(np.prod(alphas[:j + 1]) for j in range(4))
    n = 40000
    out, _ = _run_trials(P, Q, n, seed=8)
    nacc = out["n_acc"]
    assert abs(nacc.mean() - expect) < 5 * nacc.std() / np.sqrt(n)


def test_equal_distributions_always_accept():
    V = 8
    g = np.random.default_rng(9)
    P = [_dirichlet(g, V) for _ in range(4)]
    out, toks = _run_trials(P, P[:3], 3000, seed=10)
    assert np.all(out["n_acc"] == 3)
    assert np.array_equal(out["tokens"][:, :3], toks)
    counts = np.bincount(out["tokens"][:, 3], minlength=V)
    _, pval = stats.chisquare(counts, 3000 * P[3])
    assert pval > 1e-4


def test_disjoint_supports_always_reject_residual_is_p():
    V = 8
    p = np.array([0.5, 0.3, 0.2, 0, 0, 0, 0, 0])
    q = np.array([0, 0, 0, 0.25, 0.25, 0.25, 0.25, 0.0])
    n = 20000
    out, _ = _run_trials([p, p], [q], n, seed=12)
    assert np.all(out["n_acc"] == 0)
    counts = np.bincount(out["tokens"][:, 0], minlength=V)
    assert np.all(counts[3:] == 0)
    _, pval = stats.chisquare(counts[:3], n * p[:3])
    assert pval > 1e-4


def test_one_hot_draft_accepts_with_p_of_x():
    V = 8
    g = np.random.default_rng(13)
    p = _dirichlet(g, V, 2.0)
    q = np.zeros(V)
    q[5] = 1.0
    n = 40000
    out, _ = _run_trials([p, p], [q], n, seed=14)
    rate = (out["n_acc"] == 1).mean()
    assert abs(rate - p[5]) < 5 * np.sqrt(p[5] * (1 - p[5]) / n)
    # on rejection the replacement never repeats the rejected token
    rej = out["n_acc"] == 0
    assert np.all(out["tokens"][rej, 0] != 5)


def test_zero_length_is_plain_sampling():
    V = 12
    g = np.random.default_rng(15)
    p = _dirichlet(g, V)
    n = 30000
    out, _ = _run_trials([p], [_dirichlet(g, V)], n, seed=16, ell=0)
    assert np.all(out["n_acc"] == 0)
    counts = np.bincount(out["tokens"][:, 0], minlength=V)
    _, pval = stats.chisquare(counts, n * p)
    assert pval > 1e-4
    assert np.all(out["tokens"][:, 1:] == -1)


def test_figure1_flow():
    """DSpark summary, Figure 1: E and F accepted, G rejected and replaced,
    three tokens out.  Constructed so every decision is forced."""
    V = 8
    E, F, G, Gp = 1, 2, 3, 6
    pE = np.full(V, 0.1); pE[E] = 0.3
    qE = np.full(V, 0.1); qE[E] = 0.3           # p = q at E -> accept
    pF = np.zeros(V); pF[F] = 1.0
    qF = np.full(V, 1.0 / V)                     # p(F) >= q(F) -> accept
    pG = np.zeros(V); pG[Gp] = 1.0               # p(G) = 0 -> reject
    qG = np.zeros(V); qG[G] = 1.0
    pH = np.full(V, 1.0 / V)
    tgt = np.stack([_logits(v / v.sum()) for v in (pE, pF, pG, pH)])
    drf = np.stack([_logits(v / v.sum()) for v in (qE, qF, qG)])
    out = Vf.verify(tgt, [0], drf, [0], np.array([[E, F, G]]), [3], V, 1.0, 77)
    assert out["n_acc"][0] == 2
    assert list(out["tokens"][0]) == [E, F, Gp, -1]


def test_degenerate_inputs():
    V = 8
    good = np.zeros(V)
    nan_row = good.copy(); nan_row[3] = np.nan
    ninf = np.full(V, -np.inf)
    # bad draft token at position 1 -> bit 1, rejected, residual sampled
    skew = good.copy(); skew[4] = 2.0
    out = Vf.verify(np.stack([skew, good]), [0], np.stack([good]), [0], [[V + 3]], [1], V, 1.0, 1)
    assert out["status"][0] == Vf.ST_BAD_TOKEN and out["n_acc"][0] == 0
    assert out["tokens"][0, 0] == 4          # residual max(0, p - q) is one-hot at 4
    # with p = q the residual is empty -> bit 8, drawn from p instead
    out = Vf.verify(np.stack([good, good]), [0], np.stack([good]), [0], [[-1]], [1], V, 1.0, 1)
    assert out["status"][0] == Vf.ST_BAD_TOKEN | Vf.ST_ZERO_RESIDUAL
    assert 0 <= out["tokens"][0, 0] < V
    # NaN in a needed row -> bit 2, request fails
    out = Vf.verify(np.stack([good, nan_row]), [0], np.stack([good]), [0], [[1]], [1], V, 1.0, 1)
    assert out["status"][0] & Vf.ST_NONFINITE
    assert out["n_acc"][0] == 0 and np.all(out["tokens"][0] == -1)
    # NaN only in a row past l_r is never read
    out = Vf.verify(np.stack([good, nan_row]), [0], np.stack([good]), [0], [[1]], [0], V, 1.0, 1)
    assert out["status"][0] == 0
    # all -inf -> bit 4
    out = Vf.verify(np.stack([ninf]), [0], np.stack([good]), [0], [[1]], [0], V, 1.0, 1)
    assert out["status"][0] == Vf.ST_ZERO_Z and out["tokens"][0, 0] == -1
    # q(x) = 0 at the draft token -> bit 16, accepted because p(x) > 0
    q0 = good.copy(); q0[2] = -np.inf
    out = Vf.verify(np.stack([good, good]), [0], np.stack([q0]), [0], [[2]], [1], V, 1.0, 1)
    assert out["status"][0] == Vf.ST_ZERO_Q and out["n_acc"][0] == 1


def test_near_boundary_bookkeeping():
    V = 8
    g = np.random.default_rng(17)
    P = [_dirichlet(g, V) for _ in range(3)]
    Q = [_dirichlet(g, V) for _ in range(2)]
    out, toks = _run_trials(P, Q, 500, seed=18)
    # recompute every recorded accept distance from its definition
    for kind, r, j, dist in out["decisions"]:
        if kind == "accept":
            x = toks[r, j - 1]
            u = rng.uniform(18, r, j, rng.DRAW_ACCEPT)
            assert np.isclose(dist, abs(u - P[j - 1][x] / Q[j - 1][x]), rtol=1e-12)
        assert dist >= 0


def _random_batch(g, R, gmax, V, close=0.7):
    """Reserved-slot rows: target N(0, 2^2), drafts near the targets, lengths
    and tokens random (some outside [0, V), some with q(x) = 0)."""
    tgt = g.normal(0, 2, (R * (gmax + 1), V))
    drf = np.empty((R * gmax, V))
    for r in range(R):
        drf[r * gmax:(r + 1) * gmax] = tgt[r * (gmax + 1):r * (gmax + 1) + gmax] + g.normal(0, close, (gmax, V))
    toks = g.integers(0, V, (R, gmax))
    toks[g.random((R, gmax)) < 0.03] = V + 1
    ell = g.integers(0, gmax + 1, R)
    return tgt, drf, toks, ell


def test_stop_at_rejection_equals_full_verification_on_usable_rows():
    """With every row usable the outcome does not depend on the rows past the
    first rejection, so both procedures give the same result."""
    g = np.random.default_rng(31)
    R, gmax, V = 60, 6, 40
    tgt, drf, toks, ell = _random_batch(g, R, gmax, V)
    for r in range(0, R, 7):                     # q(x) = 0 at some draft tokens
        drf[r * gmax, min(toks[r, 0], V - 1)] = -np.inf
    t0, d0 = np.arange(R) * (gmax + 1), np.arange(R) * gmax
    for T in (1.0, 0.6):
        a = Vf.verify(tgt, t0, drf, d0, toks, ell, V, T, 5)
        b = Vf.verify_until_rejection(tgt, t0, drf, d0, toks, ell, V, T, 5)
        assert np.array_equal(a["n_acc"], b["n_acc"])
        assert np.array_equal(a["tokens"], b["tokens"])
        assert np.array_equal(a["status"], b["status"])
        assert a["decisions"] == b["decisions"]
        for r in range(R):
            n = b["n_acc"][r]
            tested = min(n + 1, ell[r])          # positions whose test ran
            assert np.array_equal(a["probe"][r, :tested], b["probe"][r, :tested])
            assert np.array_equal(a["drf_stats"][r, :tested], b["drf_stats"][r, :tested])
            assert np.array_equal(a["tgt_stats"][r, :tested], b["tgt_stats"][r, :tested])
            assert np.all(b["probe"][r, tested:] == 0)


def test_stop_at_rejection_never_reads_past_the_rejection():
    """Rows past each request's first rejection replaced by NaN / all -inf:
    the result is that of the clean rows; an unusable row at or before the
    rejection (or an unusable bonus row after full acceptance) fails the
    request, as verify() does."""
    g = np.random.default_rng(32)
    R, gmax, V = 40, 5, 30
    tgt, drf, toks, ell = _random_batch(g, R, gmax, V, close=1.5)
    t0, d0 = np.arange(R) * (gmax + 1), np.arange(R) * gmax
    clean = Vf.verify(tgt, t0, drf, d0, toks, ell, V, 1.0, 9)
    bad_t, bad_d = tgt.copy(), drf.copy()
    spoiled = 0
    for r in range(R):
        n, L = clean["n_acc"][r], ell[r]
        if n < L:                                # rejected at position n + 1
            bad_t[t0[r] + n + 1:t0[r] + L + 1] = np.nan
            bad_d[d0[r] + n + 1:d0[r] + L] = -np.inf
            spoiled += L - n
    assert spoiled > 20
    lazy = Vf.verify_until_rejection(bad_t, t0, bad_d, d0, toks, ell, V, 1.0, 9)
    for k in ("n_acc", "tokens", "status"):
        assert np.array_equal(lazy[k], clean[k]), k
    full = Vf.verify(bad_t, t0, bad_d, d0, toks, ell, V, 1.0, 9)
    assert np.any(full["status"] & Vf.ST_NONFINITE)   # the full procedure reads them
    # an unusable row at the rejected position itself, and a bad bonus row
    r = next(r for r in range(R) if clean["n_acc"][r] < ell[r])
    j = clean["n_acc"][r] + 1
    t2 = tgt.copy(); t2[t0[r] + j - 1, 0] = np.nan
    out = Vf.verify_until_rejection(t2, t0, drf, d0, toks, ell, V, 1.0, 9)
    assert out["status"][r] == Vf.ST_NONFINITE and out["n_acc"][r] == 0 and np.all(out["tokens"][r] == -1)
    r = next(r for r in range(R) if clean["n_acc"][r] == ell[r])
    t3 = tgt.copy(); t3[t0[r] + ell[r]] = -np.inf
    out = Vf.verify_until_rejection(t3, t0, drf, d0, toks, ell, V, 1.0, 9)
    assert out["status"][r] & Vf.ST_ZERO_Z and np.all(out["tokens"][r] == -1)
