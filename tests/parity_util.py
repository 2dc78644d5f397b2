"""Helpers for GPU-vs-oracle parity checks (used by the GPU tests and the smoke check).

Decisions whose oracle-side distance to the threshold is below NEAR (in units
of the uniform) are "near-boundary": the GPU works from fp32 row statistics and
may legitimately land on the other side of such a threshold.  Every other
decision must agree exactly, and the decisions that do diverge are counted
(the tests bound their number).  With flat distributions over ~1e5 tokens a
single token spans only ~1e-5 of the unit interval, so near-boundary decisions
themselves are common there; divergences are not.
"""

import numpy as np
import torch

from oracle import verify as OV

NEAR = 1e-6
REL = 1e-5
# probe_probs are fp32: below 2^-126 they are subnormal and keep an absolute
# precision of 2^-149, so they are compared to within that as well
FP32_TINY = 2.0 ** -149


def to_np(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def oracle_verify_subset(inp, reqs, ell, stop_at_rejection=False):
    """Oracle verification of requests `reqs` of a reserved-slot-layout input,
    keeping their true request indices for the uniforms.  Only the rows of
    those requests are copied to the host.  stop_at_rejection: the oracle
    that reads positions in order and stops at the first rejection."""
    V = inp["V"]
    t0 = to_np(inp["tgt_row0"]).astype(np.int64)
    d0 = to_np(inp["drf_row0"]).astype(np.int64)
    toks = to_np(inp["draft_tokens"])
    ell = np.asarray(ell)
    tgt_rows, drf_rows, tr0, dr0 = [], [], [], []
    for r in reqs:
        L = int(ell[r])
        tr0.append(len(tgt_rows))
        tgt_rows.extend(range(int(t0[r]), int(t0[r]) + L + 1))
        dr0.append(len(drf_rows))
        drf_rows.extend(range(int(d0[r]), int(d0[r]) + L))

    def gather(t, rows):
        if not rows:
            return np.zeros((1, V))
        idx = torch.as_tensor(rows, dtype=torch.long, device=t.device)
        return to_np(t.index_select(0, idx)[:, :V]).astype(np.float64)

    tgt = gather(inp["tgt"], tgt_rows)
    drf = gather(inp["drf"], drf_rows)
    pos0 = None if inp.get("pos0") is None else to_np(inp["pos0"])[list(reqs)]
    fn = OV.verify_until_rejection if stop_at_rejection else OV.verify
    return fn(tgt, np.array(tr0), drf, np.array(dr0), toks[list(reqs)], ell[list(reqs)],
              V, inp["temperature"], inp["seed"], pos0, req_ids=list(reqs))


def oracle_verify_all(inp, ell, reqs=None, chunk=32):
    """oracle_verify_subset over every request of `reqs` (default: all),
    taken `chunk` requests at a time so that only that many requests' rows
    are on the host at once; the per-request outputs of the chunks are
    concatenated in request order (row i is request reqs[i]) and the
    decisions carry their position i in that order."""
    reqs = list(range(inp["R"])) if reqs is None else [int(r) for r in reqs]
    parts = []
    for c0 in range(0, len(reqs), chunk):
        ora = oracle_verify_subset(inp, reqs[c0:c0 + chunk], ell)
        ora["decisions"] = [(kind, c0 + i, j, d) for kind, i, j, d in ora["decisions"]]
        parts.append(ora)
    out = {k: np.concatenate([o[k] for o in parts]) for k in
           ("n_acc", "tokens", "status", "probe", "tgt_stats", "drf_stats", "alpha")}
    out["decisions"] = [d for o in parts for d in o["decisions"]]
    return out


class DecisionTally:
    """Verify decisions compared in a test session: all of them, those the
    oracle marks near-boundary, and those where the GPU decided otherwise
    (each of which compare_verify has already required to be near-boundary).
    Divergences are bounded over the whole session: at most 0.01 % of the
    decisions (the parity bar for token decisions)."""

    MAX_DIVERGED = 1e-4

    def __init__(self):
        self.rows = []

    def add(self, what, n_dec, n_near, n_div):
        self.rows.append((what, n_dec, n_near, n_div))

    def totals(self):
        return tuple(sum(r[i] for r in self.rows) for i in (1, 2, 3))

    def check(self):
        n_dec, n_near, n_div = self.totals()
        assert n_div <= self.MAX_DIVERGED * n_dec, (
            f"{n_div} of {n_dec} verify decisions diverged from the oracle "
            f"(bound {self.MAX_DIVERGED * n_dec:.2f})")
        return n_dec, n_near, n_div


VERIFY_TALLY = DecisionTally()


def compare_verify(gpu, ora, reqs):
    """n_acc and tokens must match exactly except for requests with a
    near-boundary decision.  Returns (decisions, near-boundary, mismatches)."""
    near = set()
    n_dec = 0
    n_near = 0
    for _kind, i, _j, dist in ora["decisions"]:
        n_dec += 1
        if dist < NEAR:
            n_near += 1
            near.add(i)
    g_nacc = to_np(gpu["n_acc"])
    g_tok = to_np(gpu["tokens"])
    g_st = to_np(gpu["status"])
    mism = 0
    for i, r in enumerate(reqs):
        same = (g_nacc[r] == ora["n_acc"][i] and np.array_equal(g_tok[r], ora["tokens"][i])
                and g_st[r] == ora["status"][i])
        if not same:
            assert i in near, (f"request {r}: gpu n_acc={g_nacc[r]} tokens={g_tok[r]} "
                               f"status={g_st[r]} vs oracle n_acc={ora['n_acc'][i]} "
                               f"tokens={ora['tokens'][i]} status={ora['status'][i]}")
            mism += 1
    return n_dec, n_near, mism


def assert_rel(a, b, rel=REL, what="", atol=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b)
    bad = err > rel * np.abs(b) + atol
    assert not np.any(bad), (f"{what}: {bad.sum()} of {bad.size} outside rel {rel}; worst "
                             f"{(err / np.maximum(np.abs(b), 1e-300)).max():.3e}")


def moved_mass(L_gpu, L_ora, V, T):
    """Probability mass (under the oracle row's normaliser) that the elements
    where two bf16 drafted rows differ move: sum |e^(L_gpu/T) - e^(L_ora/T)|
    / sum e^(L_ora/T).  Returns (moved, oracle log-normaliser, m, Z) or
    None for a row without a finite normaliser."""
    _, m_o, Z_o, st = OV.row_softmax(L_ora, V, T)
    if st:
        return None
    L_gpu = np.asarray(L_gpu[:V], np.float64)
    L_ora = np.asarray(L_ora[:V], np.float64)
    lse_o = m_o + np.log(Z_o)
    diff = L_gpu != L_ora
    moved = float(np.sum(np.abs(np.exp(L_gpu[diff] / T - lse_o) - np.exp(L_ora[diff] / T - lse_o))))
    dm = float(np.max(np.abs(L_gpu[diff] - L_ora[diff]))) / T if diff.any() else 0.0
    return moved, lse_o, m_o, dm


def cdf_shift(L_gpu, L_ora, V, T):
    """Bound on |F_gpu - F_ora| over the vocabulary for the inverse CDFs of
    two drafted rows: the cumulative sums differ by at most the moved mass
    and so do the normalisers, so 2 * moved / (1 - moved)."""
    mm = moved_mass(L_gpu, L_ora, V, T)
    if mm is None or mm[0] >= 0.5:
        return np.inf
    return 2.0 * mm[0] / (1.0 - mm[0])


def check_examined_stats(gpu, ora, reqs, ell, gmax):
    """As check_stats for verification that stops at the first rejection:
    the rows and positions the oracle examined (up to each request's decided
    position), which the GPU has read too."""
    rs = to_np(gpu["row_stats"])
    pr = to_np(gpu["probe"])
    g_nacc = to_np(gpu["n_acc"])
    for i, r in enumerate(reqs):
        if ora["status"][i] & (OV.ST_NONFINITE | OV.ST_ZERO_Z):
            continue
        # rows both sides examined (they differ only after a near-boundary
        # divergence, which compare_verify has vetted)
        L, n = int(ell[r]), min(int(ora["n_acc"][i]), int(g_nacc[r]))
        tmax = n if n < L else L             # target slots read: 0..tmax
        dmax = n + 1 if n < L else L         # draft positions read: 1..dmax
        assert_row_stats(rs[r, :tmax + 1], ora["tgt_stats"][i, :tmax + 1], f"r{r} target rows")
        assert_row_stats(rs[r, gmax + 1:gmax + 1 + dmax], ora["drf_stats"][i, :dmax], f"r{r} draft rows")
        ok = ora["probe"][i, :dmax, 1] > 0
        assert_rel(pr[r, :dmax][ok], ora["probe"][i, :dmax][ok], what=f"r{r} probe p,q", atol=FP32_TINY)


def check_drafted_row_stats(mz_gpu, L_gpu, L_ora, V, T, what=""):
    """(m, Z) that a drafting head reported for its bf16 row L_gpu against the
    oracle's (m, Z) of its own row L_ora.  The rows differ only where a logit
    rounds the other way (each such element is held to the logits tolerance
    separately), so the normaliser may move by exactly the mass those
    elements move: |Z_gpu e^m_gpu / (Z_ora e^m_ora) - 1| <= REL + that mass,
    and m by REL plus the largest such move.  Rows without such elements are
    held to REL."""
    mm = moved_mass(L_gpu, L_ora, V, T)
    if mm is None:
        return
    moved, lse_o, m_o, dm = mm
    m_g, Z_g = float(mz_gpu[0]), float(mz_gpu[1])
    rel = abs(np.expm1(m_g + np.log(Z_g) - lse_o))
    assert rel <= REL + moved, f"{what}: normaliser off by {rel:.3e} (rows differ by mass {moved:.3e})"
    assert abs(m_g - m_o) <= REL * max(1.0, abs(m_o)) + dm, f"{what}: m {m_g} vs {m_o}"


def assert_row_stats(got, ref, what):
    """(m, Z) pairs of rows: m = max/T within REL (relative and absolute), and
    the normaliser e^m * Z within REL relative.  A reported Z is taken
    relative to the reported, fp32-rounded m, so the pair is compared as the
    normaliser it stands for rather than Z alone."""
    got = np.asarray(got, np.float64).reshape(-1, 2)
    ref = np.asarray(ref, np.float64).reshape(-1, 2)
    assert_rel(got[:, 0], ref[:, 0], what=f"{what} m", atol=REL)
    lse_err = np.abs(np.expm1((got[:, 0] + np.log(got[:, 1])) - (ref[:, 0] + np.log(ref[:, 1]))))
    assert np.all(lse_err <= REL), f"{what} normaliser e^m Z: worst relative error {lse_err.max():.3e}"


def check_stats(gpu, ora, reqs, ell, gmax, draft=True):
    """(m, Z) per batch row and (p(x), q(x)) per tested position, rel 1e-5
    (draft=False: target rows and p(x) only)."""
    rs = to_np(gpu["row_stats"])
    pr = to_np(gpu["probe"])
    for i, r in enumerate(reqs):
        L = int(ell[r])
        if ora["status"][i] & (OV.ST_NONFINITE | OV.ST_ZERO_Z):
            if gpu.get("alpha") is not None:
                assert np.all(to_np(gpu["alpha"])[r] == 0)   # a failed request accepts nothing
            continue
        assert_row_stats(rs[r, :L + 1], ora["tgt_stats"][i, :L + 1], f"r{r} target rows")
        if draft:
            assert_row_stats(rs[r, gmax + 1:gmax + 1 + L], ora["drf_stats"][i, :L], f"r{r} draft rows")
            ok = ora["probe"][i, :L, 1] > 0
            assert_rel(pr[r, :L][ok], ora["probe"][i, :L][ok], what=f"r{r} probe p,q", atol=FP32_TINY)
        else:
            assert_rel(pr[r, :L, 0], ora["probe"][i, :L, 0], what=f"r{r} probe p", atol=FP32_TINY)
        if gpu.get("alpha") is not None:
            al = to_np(gpu["alpha"])
            assert_rel(al[r, :L], ora["alpha"][i, :L], what=f"r{r} alpha", atol=1e-7)
            assert np.all(al[r, L:] == 0)


def compare_draft_chains(gpu_tokens, gpu_conf, ref, reqs, check_logits=None, shift=None):
    """A drafted block from the GPU against the oracle's own chain, run from
    the same seeded inputs (no GPU output enters the oracle).

    ref holds tokens, conf and dists [n][gamma] for the requests `reqs` (row i
    is request reqs[i]).  Each request is walked position by position while
    the two chains share their history: the confidence must agree within
    REL, check_logits(i, r, k) (if given) checks that position's logits, and
    the tokens must be equal unless the oracle's draw lies within NEAR plus
    shift(i, r, k) of a boundary, where the chains may part; shift (if given)
    bounds how far the two drafted rows' inverse CDFs can lie apart (the rows
    differ where a logit rounds the other way, within the logits tolerance).
    What follows a parting is drawn from another history and is not
    compared.  Returns (near-boundary draws, partings, positions compared,
    set of requests that parted)."""
    gpu_tokens = np.asarray(gpu_tokens)
    gpu_conf = np.asarray(gpu_conf)
    near = compared = 0
    parted = set()
    for i, r in enumerate(reqs):
        for k in range(gpu_tokens.shape[1]):
            compared += 1
            assert_rel(gpu_conf[r, k], ref["conf"][i, k], what=f"conf r{r} k{k + 1}")
            if check_logits is not None:
                check_logits(i, r, k)
            is_near = bool(ref["dists"][i, k] < NEAR)
            near += is_near
            if gpu_tokens[r, k] != ref["tokens"][i, k]:
                sh = shift(i, r, k) if shift is not None else 0.0
                assert sh < 1e-3, f"r{r} k{k + 1}: drafted rows differ by {sh:.3e} of their mass"
                assert ref["dists"][i, k] < NEAR + sh, (
                    f"r{r} k{k + 1}: gpu token {gpu_tokens[r, k]} vs oracle {ref['tokens'][i, k]} "
                    f"(oracle distance {ref['dists'][i, k]:.3e}, rows' CDFs within {sh:.3e})")
                parted.add(r)
                break
    return near, len(parted), compared, parted


def partings_bound(compared):
    """Most chains that may part among `compared` positions.  Each drafted
    row is a bf16 rounding of an fp32-accumulated sum, so a logit can round
    the other way from the oracle's (within the logits tolerance); every
    parting must be explained by that (asserted draw by draw), and partings
    stay rare: at most 0.75 % of the positions compared (at least one)."""
    return max(1, int(np.ceil(0.0075 * compared)))


def bf16_half_ulp(y):
    """Half a bf16 unit in the last place of each value (normal range)."""
    _, e = np.frexp(y)
    e = np.maximum(e, -125)
    return np.ldexp(0.5, e - 8)
