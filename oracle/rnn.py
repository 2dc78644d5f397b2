"""RNN sequential drafting head (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (DSpark summary, "innovation one": the light sequential head
on top of the parallel backbone comes in two forms, a Markov head that only
sees the previous token through a low-rank table, and an RNN head that keeps
a recurrent state to capture longer dependencies; Figure 1 for the anchor):

* a recurrent state over the block, s_k = tanh(W s_{k-1} + E_s[x_{k-1}]),
  s_0 = 0, fed by the previously drafted token (the anchor x_0 first);
* position k's draft distribution P_k = softmax(U_k + s_k . C), a low-rank
  readout C (d x V) of the state added to the backbone logits;
* sampling, confidence and degenerate cases exactly as the Markov head
  (``markov.draw_position``).

Readings (all listed in the design notes; the page gives no formula for this
head): an Elman recurrence with tanh, no biases, zero initial state, weights
shared across positions; the state and the readout are exact (fp64) before
the one bf16 rounding of the logits; an anchor outside [0, V) contributes no
embedding term (and sets status bit 1, as for the Markov head).

Pins (tests/test_oracle_rnn.py): torch.nn.RNNCell with one-hot inputs for the
state, the W = 0 reduction to a previous-token table (tanh(E_s[x]) . C), the
C = 0 reduction to independent softmax(U_k) draws, and an exact joint
enumeration of a small chain against Monte-Carlo frequencies.
"""

import numpy as np

from .markov import draw_position
from .verify import ST_BAD_TOKEN


def rnn_state(W, E_s, s_prev, x_prev):
    """s = tanh(W s_prev + E_s[x_prev]) per row, fp64; no embedding term for
    an x_prev outside [0, V)."""
    E_s = np.asarray(E_s, np.float64)
    V = E_s.shape[0]
    x_prev = np.asarray(x_prev, np.int64)
    valid = (x_prev >= 0) & (x_prev < V)
    emb = np.where(valid[:, None], E_s[np.where(valid, x_prev, 0)], 0.0)
    return np.tanh(np.asarray(s_prev, np.float64) @ np.asarray(W, np.float64).T + emb)


def rnn_step(U_k, W, E_s, C, s_prev, x_prev, h_k, E, w, T, seed, req_ids, pos):
    """One block position for a set of requests: returns (state s[n][d],
    pre-rounding logits y[n][V], rounded L, tokens, conf, status, dists)."""
    U_k = np.asarray(U_k, np.float64)
    V = U_k.shape[1]
    x_prev = np.asarray(x_prev, np.int64)
    status = np.where((x_prev >= 0) & (x_prev < V), 0, ST_BAD_TOKEN).astype(np.int32)
    s = rnn_state(W, E_s, s_prev, x_prev)
    y = U_k + s @ np.asarray(C, np.float64)
    L, tokens, conf, status, dists = draw_position(y, x_prev, h_k, E, w, T, seed, req_ids, pos,
                                                   status)
    return s, y, L, tokens, conf, status, dists


def rnn_draft(U, W, E_s, C, x0, h, E, w, T, seed, pos0=None):
    """Draft a whole block for every request.  U[R][gamma][V], W[d][d],
    E_s[V][d], C[d][V], x0[R], h[R][gamma][H], E[V][re], w[H + re].
    Returns a dict: tokens, L, y, s (states [R][gamma][d]), conf, status,
    dists."""
    U = np.asarray(U)
    R, gamma, V = U.shape
    d = np.asarray(W).shape[0]
    pos0 = np.zeros(R, np.int64) if pos0 is None else np.asarray(pos0, np.int64)
    out = {"tokens": np.zeros((R, gamma), np.int64), "L": np.zeros((R, gamma, V)),
           "y": np.zeros((R, gamma, V)), "s": np.zeros((R, gamma, d)), "conf": np.zeros((R, gamma)),
           "status": np.zeros(R, np.int32), "dists": np.zeros((R, gamma))}
    s = np.zeros((R, d))
    x_prev = np.asarray(x0, np.int64).copy()
    req = np.arange(R)
    for k in range(1, gamma + 1):
        s, y, Lk, tok, c, st, dist = rnn_step(U[:, k - 1], W, E_s, C, s, x_prev, h[:, k - 1], E, w, T,
                                              seed, req, pos0 + k)
        out["s"][:, k - 1] = s
        out["y"][:, k - 1] = y
        out["L"][:, k - 1] = Lk
        out["tokens"][:, k - 1] = tok
        out["conf"][:, k - 1] = c
        out["dists"][:, k - 1] = dist
        out["status"] |= st
        x_prev = tok
    return out
