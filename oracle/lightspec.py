"""Training-free two-stage budget planner (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (LightSpec article: the two optimisation stages, the
runtime statistics kept as exponential moving averages, interpolation across
draft lengths for configurations with too few samples, the runtime cost
tables):

* an EMA table of the per-position acceptance rate, fed after every verify
  step by the acceptance probabilities alpha[r, j] = sum_v min(p, q) that
  verification reports (DSpark summary, "2.1": the same quantity is the
  confidence head's label);
* confidences for planning: the EMA value of each position, with positions
  never observed filled by linear interpolation between the nearest observed
  positions (held constant beyond the first / last observed one);
* stage 1 (verify budget): the hardware-aware prefix scheduler (global argmax
  of Theta = tau * SPS(B), as in ``schedule``) run on those confidences, the
  same for every request, over the previous round's draft lengths;
* stage 2 (draft budget): for every candidate draft length d of the next
  round, the best verify batch when every request drafts d tokens, and the
  expected decode throughput
      Phi(d) = (R + tau*(d)) / (draft_cost[d-1] + 1 / SPS(B*(d)))
  (one emitted token per request beyond the accepted ones, per cycle of
  drafting d tokens and verifying B*(d) rows); the next round drafts the
  smallest d maximising Phi.

Readings (the article fixes none of the formulas; all listed in the design
notes): statistics are kept per draft position only; the batch mean of a
step counts every verified position j <= l_r of every request that did not
fail; the first observation of a position replaces its prior; the update is
e <- (1 - lam) * e + lam * mean, in fp64, sums in request order; SPS(B) is
verify passes per unit time and draft_cost[d-1] the time of drafting d tokens
for the whole batch, in the same unit; stage 2 considers d = 1..gamma_max.

Pins (tests/test_oracle_lightspec.py): numpy's masked mean, the closed form of
an EMA driven by a constant mean, exact reproduction of a linear table by the
interpolation, an exhaustive search over every prefix-length vector for both
stages, and the closed form of Phi for a constant throughput table.
"""

import numpy as np

from . import schedule as S
from .verify import ST_NONFINITE, ST_ZERO_Z


def ema_update(alpha, ell, status, lam, ema, count):
    """Fold one verify step into the per-position EMA table.

    alpha [R][G] (fp32 values), ell [R], status [R]; ema [G] fp64 and count [G]
    int64 are the state.  Returns the new (ema, count)."""
    alpha = np.asarray(alpha, dtype=np.float32)
    R, G = alpha.shape
    ema = np.array(ema, dtype=np.float64).copy()
    count = np.array(count, dtype=np.int64).copy()
    lam = float(lam)
    for j in range(1, G + 1):
        total, n = 0.0, 0
        for r in range(R):
            if int(status[r]) & (ST_NONFINITE | ST_ZERO_Z):
                continue
            if min(max(int(ell[r]), 0), G) >= j:
                total += float(alpha[r, j - 1])
                n += 1
        if n == 0:
            continue
        mean = total / n
        if count[j - 1] == 0:
            ema[j - 1] = mean
        else:
            ema[j - 1] = (1.0 - lam) * float(ema[j - 1]) + lam * mean
        count[j - 1] += n
    return ema, count


def planning_confidences(ema, count):
    """Per-position confidences for planning, fp64 before rounding: observed
    positions keep their EMA value; unobserved ones are interpolated linearly
    between the nearest observed neighbours, held constant past the ends;
    with nothing observed the table (the caller's prior) is used as is."""
    ema = np.asarray(ema, dtype=np.float64)
    count = np.asarray(count, dtype=np.int64)
    G = ema.shape[0]
    seen = [j for j in range(G) if count[j] > 0]
    out = np.zeros(G, dtype=np.float64)
    for j in range(G):
        if not seen or count[j] > 0:
            out[j] = ema[j]
            continue
        below = [s for s in seen if s < j]
        above = [s for s in seen if s > j]
        if not below:
            out[j] = ema[above[0]]
        elif not above:
            out[j] = ema[below[-1]]
        else:
            lo, hi = below[-1], above[0]
            t = float(j - lo) / float(hi - lo)
            out[j] = float(ema[lo]) + (float(ema[hi]) - float(ema[lo])) * t
    return out


def conf_hat(ema, count):
    """The planning confidences as fp32 in [0, 1]."""
    return np.clip(planning_confidences(ema, count), 0.0, 1.0).astype(np.float32)


def plan(ema, count, d_prev, sps, draft_cost):
    """Both stages.  d_prev [R] (the previous round's draft lengths, clamped
    to [0, G]), sps fp32, draft_cost [G] fp32.  Returns a dict: conf [G]
    (fp32), stage 1 (the scheduler's result on the broadcast confidences:
    ell, B, n_sel, theta), stage 2 (phi [G], n_best [G], d_next, b_next)."""
    c = conf_hat(ema, count)
    G = c.shape[0]
    d_prev = np.asarray(d_prev, dtype=np.int64)
    R = d_prev.shape[0]
    sps = np.asarray(sps, dtype=np.float32)
    draft_cost = np.asarray(draft_cost, dtype=np.float32)

    stage1 = S.schedule(np.tile(c, (R, 1)), sps, S.GLOBAL_ARGMAX, np.clip(d_prev, 0, G))
    if R == 0 or G == 0:
        return {"conf": c, "ell": stage1["ell"], "B": stage1["B"], "n_sel": stage1["n_sel"],
                "theta": stage1["theta"], "phi": np.zeros(G), "n_best": np.zeros(G, np.int64),
                "d_next": 0, "b_next": R}

    # Stage 2.  Every request has the same survivals a_1 >= a_2 >= ..., so the
    # sorted candidates are a_1 (R times), a_2 (R times), ...: the first n of
    # them sum to T_n in fixed point whatever the order among equal values.
    a = S.survival(c[None, :])[0]
    q = [S.fixed_point(float(x)) for x in a]
    T = [0]
    for n in range(1, R * G + 1):
        T.append(T[-1] + q[(n - 1) // R])
    theta = [0.0] + [float(np.float64(T[n] * 2.0 ** -32) * np.float64(sps[R + n - 1]))
                     for n in range(1, R * G + 1)]
    phi = np.zeros(G, dtype=np.float64)
    n_best = np.zeros(G, dtype=np.int64)
    for d in range(1, G + 1):
        best = 0
        for n in range(1, R * d + 1):
            if theta[n] > theta[best]:
                best = n
        n_best[d - 1] = best
        tau = T[best] * 2.0 ** -32
        with np.errstate(divide="ignore", invalid="ignore"):   # IEEE: 1/0 = inf, Phi = 0
            t_verify = np.float64(1.0) / np.float64(sps[R + best - 1])
            phi[d - 1] = np.float64(R + tau) / (np.float64(draft_cost[d - 1]) + t_verify)
    d_next = 1
    for d in range(2, G + 1):
        if phi[d - 1] > phi[d_next - 1]:
            d_next = d
    return {
        "conf": c,
        "ell": stage1["ell"], "B": stage1["B"], "n_sel": stage1["n_sel"], "theta": stage1["theta"],
        "phi": phi, "n_best": n_best, "d_next": d_next, "b_next": R + int(n_best[d_next - 1]),
    }
