"""Lossless verification by rejection sampling (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (speculative-decoding history page, "1.1 mechanism"):
the target gives p(x) at every drafted position in one parallel pass; draft
token x with draft probability q(x) is accepted outright when p(x) >= q(x) and
otherwise with probability p(x)/q(x); after the first rejection every later
draft is discarded and the target supplies one more token.  The output law is
then exactly the target's.

Readings of the pages (all listed in the design notes):
  * the garbled comparison is read as accept iff u * q(x) < p(x) with u the
    accept uniform, i.e. probability min(1, p/q); strict, so p = 0 rejects;
  * the page does not print the law of the replacement token; losslessness
    forces it: P(x) = min(p, q)(x) + (1 - sum min(p, q)) r(x) = p(x) gives
    r = max(0, p - q) / sum max(0, p - q);
  * when all l_r drafts pass, the extra token is drawn from the target row
    after the last draft (the verify batch carries 1 + l_r target rows per
    request, DSpark summary "2.2", B = sum_r (1 + l_r));
  * sampling from weights w uses the inverse CDF in vocabulary order:
    token = min{v : cumsum(w)_v > u * sum(w)}; if rounding leaves no such v,
    the last v with w_v > 0;
  * probabilities are softmax(logits / T) in fp64 from the exact inputs.

Degenerate inputs (defined behaviour, mirrored by the GPU path):
  * draft token outside [0, V) at a verified position: status bit 1, the
    position counts as rejected;
  * a needed row (target rows 0..l_r, draft rows 1..l_r) holding NaN or +inf:
    bit 2; every logit -inf (Z = 0): bit 4.  Either fails the request:
    n_acc = 0 and all its output tokens are -1;
  * residual mass 0 after a rejection: bit 8, the token is drawn from p;
  * q(x) = 0 at a tested draft token: bit 16 (the test then accepts iff p > 0).

Near-boundary bookkeeping: every decision records its distance to the
threshold, |u - p/q| for an accept test and the gap between u * sum(w) and the
nearest cumulative-sum boundary over sum(w) for a sample.

verify_until_rejection() takes the positions in order and stops at the
first rejection; it never reads a row past it (pinned against verify(): the
same result on usable rows, and rows past the rejection replaced by NaN or
all -inf change nothing).

Pins: sum min(p, q) = 1 - TV(p, q) accept frequency, chi-square losslessness,
E[n_acc] = sum_j prod_{i<=j} alpha_i, the special cases p = q, disjoint
supports, one-hot q, l = 0 (tests/test_oracle_verify.py).
"""

import numpy as np

from .rng import uniform, DRAW_ACCEPT, DRAW_CORRECT

ST_BAD_TOKEN = 1
ST_NONFINITE = 2
ST_ZERO_Z = 4
ST_ZERO_RESIDUAL = 8
ST_ZERO_Q = 16


def row_softmax(row, V, T):
    """(probabilities, m, Z, status bits) of softmax(row[:V] / T) in fp64."""
    x = np.asarray(row[:V], dtype=np.float64)
    if np.any(np.isnan(x)) or np.any(x == np.inf):
        return None, np.nan, np.nan, ST_NONFINITE
    x = x / T
    m = x.max()
    if m == -np.inf:
        return None, m, 0.0, ST_ZERO_Z
    e = np.exp(x - m)
    Z = e.sum()
    return e / Z, m, Z, 0


def inverse_cdf(w, u):
    """Token = min{v : cumsum(w)_v > u * sum(w)}, with its boundary distance."""
    cum = np.cumsum(w)
    S = cum[-1]
    target = u * S
    tok = int(np.searchsorted(cum, target, side="right"))
    if tok >= len(w):
        tok = int(np.nonzero(w > 0)[0][-1])
    lo = cum[tok - 1] if tok > 0 else 0.0
    dist = min(abs(target - lo), abs(cum[tok] - target)) / S
    return tok, dist


def verify(tgt, tgt_row0, drf, drf_row0, draft_tokens, ell, V, T, seed, pos0=None, req_ids=None):
    """Run verification for every request.

    tgt / drf: 2-D arrays of logit rows (values exactly as the kernel sees
    them, any float dtype); request r's target row for position j (1-based,
    the row that scores x_j) is tgt[tgt_row0[r] + j - 1] and its draft row is
    drf[drf_row0[r] + j - 1].  draft_tokens[r][j-1] = x_j.

    Returns a dict of numpy arrays: n_acc[R], tokens[R][gmax+1] (-1 padded),
    status[R] (bit-or per request), probe[R][gmax][2] = (p_j(x_j), q_j(x_j)),
    tgt_stats[R][gmax+1][2] and drf_stats[R][gmax][2] = (m, Z), alpha[R][gmax],
    and decisions: a list of (kind, r, j, distance) for every accept test and
    every sample drawn.  req_ids[i] is the request index that keys request
    i's uniforms (default i), so a subset of a larger batch can be checked.
    """
    R = len(ell)
    gmax = np.asarray(draft_tokens).shape[1]
    pos0 = np.zeros(R, np.int64) if pos0 is None else np.asarray(pos0, np.int64)
    rid = np.arange(R) if req_ids is None else np.asarray(req_ids, np.int64)
    n_acc = np.zeros(R, np.int32)
    tokens = np.full((R, gmax + 1), -1, np.int32)
    status = np.zeros(R, np.int32)
    probe = np.zeros((R, gmax, 2))
    tgt_stats = np.zeros((R, gmax + 1, 2))
    drf_stats = np.zeros((R, gmax, 2))
    alpha = np.zeros((R, gmax))
    decisions = []

    for r in range(R):
        L = int(ell[r])
        p_rows, q_rows = [], []
        st = 0
        for j in range(1, L + 2):  # target rows for positions 1..L+1
            p, m, Z, s = row_softmax(tgt[tgt_row0[r] + j - 1], V, T)
            st |= s
            p_rows.append(p)
            tgt_stats[r, j - 1] = (m, Z)
        for j in range(1, L + 1):  # draft rows for positions 1..L
            q, m, Z, s = row_softmax(drf[drf_row0[r] + j - 1], V, T)
            st |= s
            q_rows.append(q)
            drf_stats[r, j - 1] = (m, Z)
        if st & (ST_NONFINITE | ST_ZERO_Z):
            status[r] = st
            continue  # failed request: n_acc = 0, tokens stay -1

        for j in range(1, L + 1):
            p, q = p_rows[j - 1], q_rows[j - 1]
            alpha[r, j - 1] = np.minimum(p, q).sum()
            x = int(draft_tokens[r][j - 1])
            if 0 <= x < V:
                probe[r, j - 1] = (p[x], q[x])

        rejected_at = 0
        for j in range(1, L + 1):
            x = int(draft_tokens[r][j - 1])
            if not (0 <= x < V):
                st |= ST_BAD_TOKEN
                rejected_at = j
                break
            p, q = p_rows[j - 1][x], q_rows[j - 1][x]
            u = uniform(seed, int(rid[r]), int(pos0[r]) + j, DRAW_ACCEPT)
            if q == 0.0:
                st |= ST_ZERO_Q
                accept = p > 0.0
                dist = np.inf
            else:
                accept = u * q < p
                dist = abs(u - p / q)
            decisions.append(("accept", r, j, dist))
            if not accept:
                rejected_at = j
                break

        if rejected_at:
            j = rejected_at
            w = np.maximum(0.0, p_rows[j - 1] - q_rows[j - 1])
            if not (w.sum() > 0.0):
                st |= ST_ZERO_RESIDUAL
                w = p_rows[j - 1]
            n = j - 1
            pos = j
        else:
            n = L
            w = p_rows[L]
            pos = L + 1
        u2 = uniform(seed, int(rid[r]), int(pos0[r]) + pos, DRAW_CORRECT)
        tok, dist = inverse_cdf(w, u2)
        decisions.append(("sample", r, pos, dist))
        n_acc[r] = n
        for j in range(1, n + 1):
            tokens[r, j - 1] = int(draft_tokens[r][j - 1])
        tokens[r, n] = tok
        status[r] = st

    return {
        "n_acc": n_acc,
        "tokens": tokens,
        "status": status,
        "probe": probe,
        "tgt_stats": tgt_stats,
        "drf_stats": drf_stats,
        "alpha": alpha,
        "decisions": decisions,
    }


def verify_until_rejection(tgt, tgt_row0, drf, drf_row0, draft_tokens, ell, V, T, seed, pos0=None,
                           req_ids=None):
    """Verification that examines each request's rows in position order and
    stops at the first rejection (speculative-decoding history page, "1.1
    mechanism": everything after the first rejection is discarded, so the
    rows past it cannot change the outcome).

    Same arguments and outputs as verify(), except: rows past the first
    rejection are never examined, so a NaN, +inf or all -inf row there fails
    nothing; a position fails the request only when its own target or draft
    row is unusable (and the bonus row only when every draft was accepted);
    probe, tgt_stats and drf_stats are filled for the rows and positions
    examined; alpha is not computed (it needs every row).  On rows that are
    all usable the result is exactly verify()'s.
    """
    R = len(ell)
    gmax = np.asarray(draft_tokens).shape[1]
    pos0 = np.zeros(R, np.int64) if pos0 is None else np.asarray(pos0, np.int64)
    rid = np.arange(R) if req_ids is None else np.asarray(req_ids, np.int64)
    n_acc = np.zeros(R, np.int32)
    tokens = np.full((R, gmax + 1), -1, np.int32)
    status = np.zeros(R, np.int32)
    probe = np.zeros((R, gmax, 2))
    tgt_stats = np.zeros((R, gmax + 1, 2))
    drf_stats = np.zeros((R, gmax, 2))
    decisions = []

    for r in range(R):
        L = int(ell[r])
        st = 0
        failed = False
        w = None
        for j in range(1, L + 1):
            p, m, Z, sp = row_softmax(tgt[tgt_row0[r] + j - 1], V, T)
            tgt_stats[r, j - 1] = (m, Z)
            q, m, Z, sq = row_softmax(drf[drf_row0[r] + j - 1], V, T)
            drf_stats[r, j - 1] = (m, Z)
            if (sp | sq) & (ST_NONFINITE | ST_ZERO_Z):
                st |= sp | sq
                failed = True
                break
            x = int(draft_tokens[r][j - 1])
            if not (0 <= x < V):
                st |= ST_BAD_TOKEN
                accept = False
            else:
                probe[r, j - 1] = (p[x], q[x])
                u = uniform(seed, int(rid[r]), int(pos0[r]) + j, DRAW_ACCEPT)
                if q[x] == 0.0:
                    st |= ST_ZERO_Q
                    accept = p[x] > 0.0
                    dist = np.inf
                else:
                    accept = u * q[x] < p[x]
                    dist = abs(u - p[x] / q[x])
                decisions.append(("accept", r, j, dist))
            if not accept:
                w = np.maximum(0.0, p - q)
                if not (w.sum() > 0.0):
                    st |= ST_ZERO_RESIDUAL
                    w = p
                n, pos = j - 1, j
                break
        if failed:
            status[r] = st
            continue
        if w is None:  # every draft accepted: the bonus row
            p, m, Z, sp = row_softmax(tgt[tgt_row0[r] + L], V, T)
            tgt_stats[r, L] = (m, Z)
            if sp & (ST_NONFINITE | ST_ZERO_Z):
                status[r] = st | sp
                continue
            w, n, pos = p, L, L + 1
        u2 = uniform(seed, int(rid[r]), int(pos0[r]) + pos, DRAW_CORRECT)
        tok, dist = inverse_cdf(w, u2)
        decisions.append(("sample", r, pos, dist))
        n_acc[r] = n
        for j in range(1, n + 1):
            tokens[r, j - 1] = int(draft_tokens[r][j - 1])
        tokens[r, n] = tok
        status[r] = st

    return {
        "n_acc": n_acc,
        "tokens": tokens,
        "status": status,
        "probe": probe,
        "tgt_stats": tgt_stats,
        "drf_stats": drf_stats,
        "alpha": None,
        "decisions": decisions,
    }
