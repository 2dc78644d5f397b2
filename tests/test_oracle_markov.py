"""Pins for the oracle's Markov drafting head and confidence head.

The exact law of a drafted block is a product of per-position softmaxes with
the previous token selecting the transition row (DSpark summary, "innovation
one").  With a full-rank table (rank = V, A_k = I) the joint law of a short
block can be enumerated exactly and compared with Monte-Carlo frequencies;
with C_k = 0 the head reduces to independent draws from softmax(U_k).
"""

import itertools

import numpy as np
from scipy import stats
from scipy.special import expit, softmax

from oracle import markov as M
from oracle import verify as Vf
from oracle.bf16 import round_to_bf16
from oracle import rng


def _eighths(g, shape, lim=4.0):
    # multiples of 1/8 in [-lim, lim]: sums of two stay exact in bf16
    return np.round(g.uniform(-lim, lim, shape) * 8) / 8


def test_full_rank_joint_enumeration():
    V, gamma, n = 6, 3, 60000
    g = np.random.default_rng(1)
    U1 = _eighths(g, (gamma, V))
    Mk = _eighths(g, (gamma, V, V))            # transition logits, row = previous token
    U = np.broadcast_to(U1, (n, gamma, V))
    A = np.broadcast_to(np.eye(V), (gamma, V, V))
    x0 = np.full(n, 2)
    H = 4
    h = np.zeros((n, gamma, H))
    E = np.zeros((V, 2))
    w = np.zeros(H + 2)
    out = M.markov_draft(U, A, Mk, x0, h, E, w, 1.0, 123)
    assert np.all(out["status"] == 0)
    # exact joint law
    probs = {}
    for seq in itertools.product(range(V), repeat=gamma):
        prev, pr = 2, 1.0
        for k, x in enumerate(seq):
            pr *= softmax(U1[k] + Mk[k, prev])[x]
            prev = x
        probs[seq] = pr
    idx = out["tokens"] @ (V ** np.arange(gamma - 1, -1, -1))
    counts = np.bincount(idx, minlength=V ** gamma)
    exp = np.array([probs[s] for s in itertools.product(range(V), repeat=gamma)]) * n
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    _, pval = stats.chisquare(obs, ex)
    assert pval > 1e-4


def test_zero_transition_is_independent_softmax_draws():
    g = np.random.default_rng(2)
    R, gamma, V, rank = 5, 4, 40, 3
    U = g.normal(0, 2, (R, gamma, V))
    A = g.normal(0, 1, (gamma, V, rank))
    C = np.zeros((gamma, rank, V))
    out = M.markov_draft(U, A, C, np.arange(R), g.normal(0, 1, (R, gamma, 8)),
                         g.normal(0, 1, (V, 3)), g.normal(0, 1, 11), 0.8, 9, pos0=np.arange(R) * 100)
    for r in range(R):
        for k in range(gamma):
            L = round_to_bf16(U[r, k])
            assert np.array_equal(out["L"][r, k], L)
            u = rng.uniform(9, r, r * 100 + k + 1, 0)
            cdf = np.cumsum(softmax(L / 0.8))
            tok = int(np.argmax(cdf > u * cdf[-1]))
            assert out["tokens"][r, k] == tok


def test_confidence_head_uses_previous_token_embedding():
    g = np.random.default_rng(3)
    R, gamma, V, rank, H, re = 3, 3, 16, 4, 8, 5
    U = g.normal(0, 1, (R, gamma, V))
    A = g.normal(0, 0.1, (gamma, V, rank))
    C = g.normal(0, 0.1, (gamma, rank, V))
    h = g.normal(0, 1, (R, gamma, H))
    E = g.normal(0, 1, (V, re))
    w = g.normal(0, 0.5, H + re)
    x0 = np.array([1, 5, 7])
    out = M.markov_draft(U, A, C, x0, h, E, w, 1.0, 4)
    prev = np.concatenate([x0[:, None], out["tokens"][:, :-1]], axis=1)
    for r in range(R):
        for k in range(gamma):
            z = float(np.dot(w, np.concatenate([h[r, k], E[prev[r, k]]])))
            assert np.isclose(out["conf"][r, k], expit(z), rtol=1e-14)


def test_bias_is_low_rank_product_of_previous_token():
    g = np.random.default_rng(4)
    R, gamma, V, rank = 4, 2, 24, 3
    U = g.normal(0, 1, (R, gamma, V))
    A = g.normal(0, 1, (gamma, V, rank))
    C = g.normal(0, 1, (gamma, rank, V))
    x0 = np.array([0, 3, 3, 23])
    out = M.markov_draft(U, A, C, x0, np.zeros((R, gamma, 2)), np.zeros((V, 1)), np.zeros(3), 1.0, 5)
    prev = np.concatenate([x0[:, None], out["tokens"][:, :-1]], axis=1)
    for r in range(R):
        for k in range(gamma):
            full = A[k] @ C[k]                 # the V x V transition table
            y = U[r, k] + full[prev[r, k]]
            assert np.allclose(out["y"][r, k], y, rtol=1e-12, atol=1e-12)


def test_invalid_anchor_and_degenerate_rows():
    V = 8
    U = np.zeros((2, 2, V))
    U[1, 0, :] = -np.inf
    A = np.ones((2, V, 2))
    C = np.ones((2, 2, V))
    out = M.markov_draft(U, A, C, np.array([V, 0]), np.zeros((2, 2, 1)), np.ones((V, 1)),
                         np.ones(2), 1.0, 1)
    assert out["status"][0] & Vf.ST_BAD_TOKEN
    assert np.array_equal(out["L"][0, 0], np.zeros(V))       # no Markov bias
    assert np.isclose(out["conf"][0, 0], 0.5)                 # no embedding term
    assert out["status"][1] & Vf.ST_ZERO_Z
    assert out["tokens"][1, 0] == -1
