"""Hardware-aware prefix scheduler (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (DSpark summary, "2.2 hardware-aware prefix scheduler";
speculative-decoding history page, DSpark "move two" and "move three"):

* survival a[r,j] = prod_{i<=j} c[r,i]: the probability that the whole draft
  prefix up to position j of request r is accepted;
* verify batch size B = sum_r (1 + l_r) and expected accepted tokens
  tau = sum_r sum_{j<=l_r} a[r,j];
* objective Theta = tau * SPS(B), SPS being a per-batch-size throughput table;
* greedy: order every candidate by survival, largest first, add them one by one
  and stop as soon as Theta starts to fall;
* asynchronous variant ("challenge 2: async scheduling and ZOS"): the capacity
  is fixed beforehand from earlier confidences and filled with the top
  candidates ranked by the current ones; without early stop the search is
  global.

Readings of the pages (all listed in the design notes):
  * survival products are taken left to right in IEEE fp32;
  * candidates are sorted by survival (not raw confidence), descending, ties by
    request then position ascending;
  * tau is accumulated in fixed point: q = rint(a * 2**32) as an integer,
    tau_n = (sum of the first n q) * 2**-32, exact in fp64;
  * Theta_n = tau_n * SPS[B_n - 1] in fp64 with B_n = R + n, Theta_0 = 0;
  * early stop: n* = (first n >= 1 with Theta_n < Theta_{n-1}) - 1, else N
    (equal Theta keeps going);
  * global argmax: the smallest n maximising Theta_n over n = 0..N;
  * capped top-K: exactly min(K, N) candidates.

Two further modes of use (DSpark summary, "2.1 confidence head": sequential
temperature scaling; experiments: confidence-threshold sweep):
  * sequential temperature scaling (STS) recalibrates every confidence before
    the survival products: c' = sigmoid(logit(c) / T_j) with one temperature
    per draft position j, read as classic temperature scaling of a binary
    probability; computed in fp64 as 1 / (1 + ((1 - c) / c) ** (1 / T_j)) and
    rounded to fp32 (c = 0 stays 0, c = 1 stays 1);
  * threshold mode keeps every candidate whose survival is at least theta:
    l_r = max{j : a[r,j] >= theta} (survival never grows along j, so this is
    the prefix of the sorted order with a >= theta).

Pins: numpy.cumprod in fp32 for the survival (closed form), a brute-force
search over every prefix-length vector for the global argmax, an independent
frontier-greedy for the early stop, the constant-SPS special case and the
Figure 1 construction; for STS scipy's expit/logit, the T = 1 identity and
the symmetries of the sigmoid; for the threshold mode the per-request
definition (tests/test_oracle_schedule.py).
"""

import numpy as np

EARLY_STOP = 0
GLOBAL_ARGMAX = 1
CAPPED_TOPK = 2
THRESHOLD = 3

FIXED_POINT_SCALE = 2.0 ** 32


def survival(conf, gamma_r=None) -> np.ndarray:
    """a[r, j-1] = fl32(a[r, j-2] * c[r, j-1]) left to right; 0 past gamma_r."""
    conf = np.asarray(conf, dtype=np.float32)
    R, gmax = conf.shape
    g = np.full(R, gmax, dtype=np.int64) if gamma_r is None else np.asarray(gamma_r, np.int64)
    a = np.zeros((R, gmax), dtype=np.float32)
    for r in range(R):
        prod = np.float32(1.0)
        for j in range(int(g[r])):
            prod = np.float32(prod * conf[r, j])
            a[r, j] = prod
    return a


def sts(conf, temps) -> np.ndarray:
    """Sequential temperature scaling: c'[r, j] = fp32(sigmoid(logit(c[r, j]) / T[j]))."""
    conf = np.asarray(conf, dtype=np.float32)
    temps = np.asarray(temps, dtype=np.float64)
    R, gmax = conf.shape
    out = np.zeros((R, gmax), dtype=np.float32)
    for r in range(R):
        for j in range(gmax):
            c = float(conf[r, j])
            if c <= 0.0:
                out[r, j] = 0.0
            elif c >= 1.0:
                out[r, j] = 1.0
            else:
                odds = (1.0 - c) / c        # exp(-logit(c))
                # a power past the fp64 range is +inf, whose sigmoid is the limit 0
                with np.errstate(over="ignore"):
                    out[r, j] = np.float32(1.0 / (1.0 + odds ** (1.0 / temps[j])))
    return out


def fixed_point(a: float) -> int:
    """q = rint(a * 2**32) as an exact integer (a is an fp32 value in [0, 1])."""
    return int(np.rint(np.float64(a) * FIXED_POINT_SCALE))


def candidates_in_order(a, gamma_r):
    """All (r, j) candidates (j 1-based) sorted by survival desc, then r, then j."""
    R = a.shape[0]
    cands = []
    for r in range(R):
        for j in range(1, int(gamma_r[r]) + 1):
            cands.append((float(a[r, j - 1]), r, j))
    cands.sort(key=lambda t: (-t[0], t[1], t[2]))
    return cands


def theta_curve(order, R, sps):
    """Theta_n for n = 0..N along the sorted order (fp64), and tau_n."""
    sps = np.asarray(sps, dtype=np.float32)
    total = 0
    thetas = [0.0]
    taus = [0.0]
    for n, (a, _r, _j) in enumerate(order, start=1):
        total += fixed_point(a)
        tau = total * (2.0 ** -32)
        taus.append(tau)
        thetas.append(float(np.float64(tau) * np.float64(sps[R + n - 1])))
    return thetas, taus


def schedule(conf, sps, mode=EARLY_STOP, gamma_r=None, cap_k=None, threshold=None,
             sts_temp=None):
    """Choose per-request verify lengths l_r.

    Returns a dict: ell[R] (int32), B, n_sel, theta (fp64 Theta at the chosen
    point), surv[R][gamma_max] (fp32), order (the sorted candidate list) and
    thetas (the Theta curve, n = 0..N).  sts_temp[gamma_max], if given,
    recalibrates the confidences first.
    """
    conf = np.asarray(conf, dtype=np.float32)
    if sts_temp is not None:
        conf = sts(conf, sts_temp)
    R, gmax = conf.shape
    g = np.full(R, gmax, dtype=np.int64) if gamma_r is None else np.asarray(gamma_r, np.int64)
    sps = np.asarray(sps, dtype=np.float32)
    a = survival(conf, g)
    order = candidates_in_order(a, g)
    N = len(order)
    if sps.shape[0] < R + N:
        raise ValueError("SPS table shorter than the largest possible batch")
    thetas, _ = theta_curve(order, R, sps)

    if mode == EARLY_STOP:
        n_sel = N
        for n in range(1, N + 1):
            if thetas[n] < thetas[n - 1]:
                n_sel = n - 1
                break
    elif mode == GLOBAL_ARGMAX:
        n_sel = 0
        for n in range(1, N + 1):
            if thetas[n] > thetas[n_sel]:
                n_sel = n
    elif mode == CAPPED_TOPK:
        if cap_k is None:
            raise ValueError("capped mode needs K")
        n_sel = min(max(int(cap_k), 0), N)
    elif mode == THRESHOLD:
        if threshold is None:
            raise ValueError("threshold mode needs theta")
        n_sel = sum(1 for (a_, _r, _j) in order if a_ >= np.float32(threshold))
    else:
        raise ValueError("unknown mode")

    ell = np.zeros(R, dtype=np.int32)
    for (_a, r, _j) in order[:n_sel]:
        ell[r] += 1
    return {
        "ell": ell,
        "B": R + n_sel,
        "n_sel": n_sel,
        "theta": thetas[n_sel],
        "surv": a,
        "order": order,
        "thetas": thetas,
    }


def async_schedule(conf, conf_prev, sps, gamma_r=None):
    """Asynchronous step: K from the previous confidences (global argmax, no
    early stop), then exactly K candidates ranked by the current ones."""
    prev = schedule(conf_prev, sps, GLOBAL_ARGMAX, gamma_r)
    cur = schedule(conf, sps, CAPPED_TOPK, gamma_r, cap_k=prev["n_sel"])
    cur["cap_k"] = prev["n_sel"]
    return cur
