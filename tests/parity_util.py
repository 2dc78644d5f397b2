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


def to_np(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def oracle_verify_subset(inp, reqs, ell):
    """Oracle verification of requests `reqs` of a reserved-slot-layout input,
    keeping their true request indices for the uniforms.  Only the rows of
    those requests are copied to the host."""
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
    return OV.verify(tgt, np.array(tr0), drf, np.array(dr0), toks[list(reqs)], ell[list(reqs)],
                     V, inp["temperature"], inp["seed"], pos0, req_ids=list(reqs))


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


def check_stats(gpu, ora, reqs, ell, gmax):
    """(m, Z) per batch row and (p(x), q(x)) per tested position, rel 1e-5."""
    rs = to_np(gpu["row_stats"])
    pr = to_np(gpu["probe"])
    for i, r in enumerate(reqs):
        L = int(ell[r])
        if ora["status"][i] & (OV.ST_NONFINITE | OV.ST_ZERO_Z):
            if gpu.get("alpha") is not None:
                assert np.all(to_np(gpu["alpha"])[r] == 0)   # a failed request accepts nothing
            continue
        assert_rel(rs[r, :L + 1, 0], ora["tgt_stats"][i, :L + 1, 0], what=f"r{r} target m", atol=REL)
        assert_rel(rs[r, :L + 1, 1], ora["tgt_stats"][i, :L + 1, 1], what=f"r{r} target Z")
        assert_rel(rs[r, gmax + 1:gmax + 1 + L, 0], ora["drf_stats"][i, :L, 0], what=f"r{r} draft m", atol=REL)
        assert_rel(rs[r, gmax + 1:gmax + 1 + L, 1], ora["drf_stats"][i, :L, 1], what=f"r{r} draft Z")
        ok = ora["probe"][i, :L, 1] > 0
        assert_rel(pr[r, :L][ok], ora["probe"][i, :L][ok], what=f"r{r} probe p,q")
        if gpu.get("alpha") is not None:
            al = to_np(gpu["alpha"])
            assert_rel(al[r, :L], ora["alpha"][i, :L], what=f"r{r} alpha", atol=1e-7)
            assert np.all(al[r, L:] == 0)
