"""Semi-autoregressive Markov drafting head plus confidence head (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (DSpark summary, "innovation one: semi-autoregressive
generation" and "2.1 confidence head"; speculative-decoding history page,
DSpark "move one"):

* a parallel backbone has already produced, for every request and every block
  position k, base logits U_k and a hidden state h_k (inputs here);
* position k's draft distribution is P_k = softmax(U_k + B_k(x_{k-1})), where
  B_k is a V x V transition table applied to the previously drafted token and
  stored low-rank as B_k(x) = A_k[x] . C_k (A_k: V x r, C_k: r x V);
* sampling is sequential over k: x_k ~ P_k, starting from the anchor x_0 that
  the target emitted (Figure 1);
* the confidence head gives c_k = sigmoid(w . [h_k ; E[x_{k-1}]]) with E the
  Markov embedding table, the estimated chance that position k is accepted
  given that every earlier one was.

Readings (all listed in the design notes):
  * the drafted logits are rounded to bf16 (ties to even) before sampling, so
    the distribution sampled is exactly the one handed to verification; the
    bias product and the add are exact (fp64) before that one rounding;
  * temperature T divides the rounded logits;
  * sampling is the inverse CDF in vocabulary order with the draw-0 uniform at
    position pos0[r] + k;
  * an anchor outside [0, V) sets status bit 1 and contributes neither Markov
    bias nor embedding term; a row whose logits hold NaN or +inf (bit 2) or are
    all -inf (bit 4) yields token -1 for that position.

Pins: the C = 0 reduction to independent softmax(U_k) draws and an exact joint
enumeration with a full-rank V x V table (r = V, A = I) against Monte-Carlo
frequencies (tests/test_oracle_markov.py).
"""

import numpy as np

from .bf16 import round_to_bf16
from .rng import uniform, DRAW_DRAFT
from .verify import inverse_cdf, ST_BAD_TOKEN, ST_NONFINITE, ST_ZERO_Z


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def markov_step(U_k, A_k, C_k, x_prev, h_k, E, w, T, seed, req_ids, pos):
    """One block position for a set of requests.

    U_k[n][V], h_k[n][H] and x_prev[n] are the rows of requests req_ids[n];
    pos[n] is the absolute position used for the draw-0 uniform.
    Returns (pre-rounding logits y[n][V] fp64, rounded logits L[n][V] fp64,
    tokens[n], conf[n], status[n], sample distances[n]).
    """
    U_k = np.asarray(U_k, np.float64)
    n, V = U_k.shape
    H = h_k.shape[1]
    x_prev = np.asarray(x_prev, np.int64)
    valid = (x_prev >= 0) & (x_prev < V)
    status = np.where(valid, 0, ST_BAD_TOKEN).astype(np.int32)
    xs = np.where(valid, x_prev, 0)

    bias_rows = np.where(valid[:, None], np.asarray(A_k, np.float64)[xs], 0.0)
    y = U_k + bias_rows @ np.asarray(C_k, np.float64)
    L, tokens, conf, status, dists = draw_position(y, x_prev, h_k, E, w, T, seed, req_ids, pos,
                                                   status)
    return y, L, tokens, conf, status, dists


def draw_position(y, x_prev, h_k, E, w, T, seed, req_ids, pos, status):
    """Shared by the sequential heads: round the exact logits y[n][V] to bf16,
    the confidence from h_k and E[x_prev], and the inverse-CDF draw.
    Returns (L, tokens, conf, status, dists)."""
    n, V = y.shape
    H = h_k.shape[1]
    x_prev = np.asarray(x_prev, np.int64)
    valid = (x_prev >= 0) & (x_prev < V)
    xs = np.where(valid, x_prev, 0)
    status = np.asarray(status, np.int32).copy()
    L = round_to_bf16(y)

    emb = np.where(valid[:, None], np.asarray(E, np.float64)[xs], 0.0)
    w = np.asarray(w, np.float64)
    z = np.asarray(h_k, np.float64) @ w[:H] + emb @ w[H:]
    conf = sigmoid(z)

    tokens = np.full(n, -1, np.int64)
    dists = np.full(n, np.inf)
    for i in range(n):
        row = L[i]
        if np.any(np.isnan(row)) or np.any(row == np.inf):
            status[i] |= ST_NONFINITE
            continue
        x = row / T
        m = x.max()
        if m == -np.inf:
            status[i] |= ST_ZERO_Z
            continue
        wts = np.exp(x - m)
        u = uniform(seed, int(req_ids[i]), int(pos[i]), DRAW_DRAFT)
        tokens[i], dists[i] = inverse_cdf(wts, u)
    return L, tokens, conf, status, dists


def markov_draft(U, A, C, x0, h, E, w, T, seed, pos0=None):
    """Draft a whole block for every request.

    U[R][gamma][V], A[gamma][V][r], C[gamma][r][V], x0[R], h[R][gamma][H],
    E[V][re], w[H + re].  Returns a dict: tokens[R][gamma], L[R][gamma][V]
    (bf16-valued fp64), y (pre-rounding fp64), conf[R][gamma], status[R],
    dists[R][gamma].
    """
    U = np.asarray(U)
    R, gamma, V = U.shape
    pos0 = np.zeros(R, np.int64) if pos0 is None else np.asarray(pos0, np.int64)
    tokens = np.zeros((R, gamma), np.int64)
    conf = np.zeros((R, gamma))
    L = np.zeros((R, gamma, V))
    Y = np.zeros((R, gamma, V))
    dists = np.zeros((R, gamma))
    status = np.zeros(R, np.int32)
    x_prev = np.asarray(x0, np.int64).copy()
    req = np.arange(R)
    for k in range(1, gamma + 1):
        y, Lk, tok, c, st, d = markov_step(
            U[:, k - 1], A[k - 1], C[k - 1], x_prev, h[:, k - 1], E, w, T, seed, req, pos0 + k)
        Y[:, k - 1] = y
        L[:, k - 1] = Lk
        tokens[:, k - 1] = tok
        conf[:, k - 1] = c
        dists[:, k - 1] = d
        status |= st
        x_prev = tok
    return {"tokens": tokens, "L": L, "y": Y, "conf": conf, "status": status, "dists": dists}
