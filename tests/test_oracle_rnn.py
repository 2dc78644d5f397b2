"""Pins for the oracle's RNN drafting head.

The state recurrence is an Elman cell with tanh (torch.nn.RNNCell with one-hot
inputs and no biases); with W = 0 the head reduces to a previous-token table
tanh(E_s[x]) . C, i.e. a Markov head; with C = 0 to independent softmax(U_k)
draws; and the joint law of a short block, with the state a deterministic
function of the drafted prefix, can be enumerated exactly.
"""

import itertools

import numpy as np
import torch
from scipy import stats
from scipy.special import softmax

from oracle import markov as M
from oracle import rnn as N
from oracle import rng
from oracle import verify as Vf
from oracle.bf16 import round_to_bf16


def test_state_is_torch_rnn_cell_with_one_hot_input():
    g = np.random.default_rng(1)
    V, d, R = 12, 5, 4
    W = g.normal(0, 0.4, (d, d))
    E_s = g.normal(0, 1, (V, d))
    cell = torch.nn.RNNCell(V, d, bias=False, nonlinearity="tanh").double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(E_s.T))
        cell.weight_hh.copy_(torch.from_numpy(W))
    s = np.zeros((R, d))
    hs = torch.zeros(R, d, dtype=torch.float64)
    for step in range(6):
        x = g.integers(0, V, R)
        s = N.rnn_state(W, E_s, s, x)
        with torch.no_grad():
            hs = cell(torch.nn.functional.one_hot(torch.from_numpy(x), V).double(), hs)
        assert np.allclose(s, hs.numpy(), rtol=0, atol=1e-14), step


def test_zero_recurrence_is_a_previous_token_table():
    g = np.random.default_rng(2)
    R, gamma, V, d, H, re = 6, 4, 30, 4, 3, 2
    U = g.normal(0, 2, (R, gamma, V))
    E_s = g.normal(0, 1, (V, d))
    C = g.normal(0, 0.5, (d, V))
    h = g.normal(0, 1, (R, gamma, H))
    E = g.normal(0, 1, (V, re))
    w = g.normal(0, 0.5, H + re)
    x0 = g.integers(0, V, R)
    out = N.rnn_draft(U, np.zeros((d, d)), E_s, C, x0, h, E, w, 0.9, 7)
    table = np.tanh(E_s)                               # A_k[x] = tanh(E_s[x]) for every k
    ref = M.markov_draft(U, np.broadcast_to(table, (gamma, V, d)), np.broadcast_to(C, (gamma, d, V)),
                         x0, h, E, w, 0.9, 7)
    assert np.allclose(out["y"], ref["y"], rtol=0, atol=1e-12)
    assert np.array_equal(out["tokens"], ref["tokens"])
    assert np.array_equal(out["conf"], ref["conf"])


def test_zero_readout_is_independent_softmax_draws():
    g = np.random.default_rng(3)
    R, gamma, V, d = 4, 5, 50, 3
    U = g.normal(0, 2, (R, gamma, V))
    out = N.rnn_draft(U, g.normal(0, 1, (d, d)), g.normal(0, 1, (V, d)), np.zeros((d, V)),
                      np.arange(R), np.zeros((R, gamma, 1)), np.zeros((V, 1)), np.zeros(2), 1.3, 11,
                      pos0=np.arange(R) * 10)
    for r in range(R):
        for k in range(gamma):
            L = round_to_bf16(U[r, k])
            u = rng.uniform(11, r, r * 10 + k + 1, 0)
            cdf = np.cumsum(softmax(L / 1.3))
            assert out["tokens"][r, k] == int(np.argmax(cdf > u * cdf[-1]))


def _eighths(g, shape, lim=3.0):
    return np.round(g.uniform(-lim, lim, shape) * 8) / 8


def test_joint_enumeration_of_a_short_block():
    V, gamma, d, n = 4, 3, 2, 60000
    g = np.random.default_rng(4)
    U1 = _eighths(g, (gamma, V))
    W = g.normal(0, 0.8, (d, d))
    E_s = g.normal(0, 1.5, (V, d))
    C = g.normal(0, 2.0, (d, V))
    x0 = 1
    out = N.rnn_draft(np.broadcast_to(U1, (n, gamma, V)), W, E_s, C, np.full(n, x0),
                      np.zeros((n, gamma, 1)), np.zeros((V, 1)), np.zeros(2), 1.0, 321)
    probs = {}
    for seq in itertools.product(range(V), repeat=gamma):
        s, prev, pr = np.zeros(d), x0, 1.0
        for k, x in enumerate(seq):
            s = np.tanh(W @ s + E_s[prev])
            pr *= softmax(round_to_bf16(U1[k] + s @ C))[x]
            prev = x
        probs[seq] = pr
    idx = out["tokens"] @ (V ** np.arange(gamma - 1, -1, -1))
    counts = np.bincount(idx, minlength=V ** gamma)
    exp = np.array([probs[s] for s in itertools.product(range(V), repeat=gamma)]) * n
    keep = exp >= 5
    _, pval = stats.chisquare(np.append(counts[keep], counts[~keep].sum()),
                              np.append(exp[keep], exp[~keep].sum()))
    assert pval > 1e-4


def test_invalid_anchor_contributes_no_embedding():
    V, d = 6, 3
    out = N.rnn_draft(np.zeros((1, 2, V)), np.eye(d), np.ones((V, d)), np.ones((d, V)), np.array([V + 2]),
                      np.zeros((1, 2, 1)), np.ones((V, 1)), np.ones(2), 1.0, 1)
    assert out["status"][0] & Vf.ST_BAD_TOKEN
    assert np.array_equal(out["s"][0, 0], np.zeros(d))       # tanh(W 0 + 0)
    assert np.array_equal(out["L"][0, 0], np.zeros(V))
