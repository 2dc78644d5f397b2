"""GPU parity of sd_markov_draft against the oracle.

The oracle runs its own sequential chain from the same seeded inputs; no GPU
output enters it.  Request by request, while the two chains share their
drafted history: each GPU bf16 logit must be a round-to-nearest of a value
within 1e-5 * sum|A_k[x]_i C_k[i, v]| (+ 1e-7 |y|, the fp32 add) of the
oracle's exact y = U + A_k[x] . C_k (fp64); the confidence and the row's
(m, Z) must match within 1e-5 relative; the tokens must be equal, except
where the oracle's draw is near-boundary (distance below 1e-6), where the
chains may part — what follows a parting is drawn from another history and
is not compared.
"""

import numpy as np
import pytest
import torch

import draft_verification_amd as sdv
from oracle import markov as OM
from oracle import schedule as OS
from oracle import verify as OV
from workloads import markov_inputs, markov_config, markov_targets
from tests.parity_util import (to_np, compare_verify, check_stats, compare_draft_chains,
                               bf16_half_ulp, partings_bound, check_drafted_row_stats, cdf_shift)

pytestmark = pytest.mark.gpu


def _run(inp, stats=True):
    out = sdv.sd_markov_draft(inp["U"], inp["A"], inp["Ct"], inp["x0"], inp["h"], inp["E"], inp["w"],
                              inp["temperature"], inp["seed"], pos0=inp.get("pos0"), stats=stats)
    torch.cuda.synchronize()
    return out


def _f(t):
    return to_np(t).astype(np.float64)


def oracle_chain(inp, reqs, keep=()):
    """The oracle's Markov chain for requests `reqs`, from the seeded inputs
    alone (the tables A_k, C_k converted once per position).  For the
    requests in `keep` it also keeps, per position, the exact logits y, the
    rounded L and the logits' tolerance."""
    T, seed, V, gamma = inp["temperature"], inp["seed"], inp["V"], inp["gamma"]
    reqs = [int(r) for r in reqs]
    n = len(reqs)
    idx = torch.as_tensor(reqs, dtype=torch.long, device=inp["U"].device)
    U = inp["U"].index_select(0, idx)
    h = inp["h"].index_select(0, idx)
    x_prev = to_np(inp["x0"])[reqs].astype(np.int64)
    pos0 = (np.zeros(n, np.int64) if inp.get("pos0") is None
            else to_np(inp["pos0"])[reqs].astype(np.int64))
    E, w = _f(inp["E"]), _f(inp["w"])
    kept = [i for i, r in enumerate(reqs) if r in set(keep)]
    ref = dict(tokens=np.zeros((n, gamma), np.int64), conf=np.zeros((n, gamma)),
               dists=np.zeros((n, gamma)), status=np.zeros(n, np.int32), y={}, L={}, tol={},
               rows=np.zeros((n, gamma, V), np.float32))
    for k in range(1, gamma + 1):
        A_k = _f(inp["A"][k - 1])
        C_k = _f(inp["Ct"][k - 1]).T
        y, L, tok, c, st, d = OM.markov_step(_f(U[:, k - 1]), A_k, C_k, x_prev, _f(h[:, k - 1]), E, w,
                                             T, seed, reqs, pos0 + k)
        if kept:
            absC = np.abs(C_k)
        for i in kept:
            xp = x_prev[i]
            terms = np.abs(A_k[xp]) @ absC if 0 <= xp < V else np.zeros(V)
            ref["y"][i, k - 1] = y[i]
            ref["L"][i, k - 1] = L[i]
            ref["tol"][i, k - 1] = bf16_half_ulp(y[i]) + 1e-5 * terms + 1e-7 * np.abs(y[i]) + 1e-30
        ref["rows"][:, k - 1] = L   # bf16 values, exact in fp32
        ref["tokens"][:, k - 1] = tok
        ref["conf"][:, k - 1] = c
        ref["dists"][:, k - 1] = d
        ref["status"] |= st
        x_prev = tok
    return ref


def check_chain(inp, out, ref, reqs):
    """Compare along the shared history; logits and (m, Z) where kept."""
    T, V = inp["temperature"], inp["V"]
    ql = out["q_logits"]
    qs = to_np(out["q_stats"]) if out.get("q_stats") is not None else None

    def check_logits(i, r, k):
        if (i, k) not in ref["y"]:
            return
        Lg = _f(ql[r, k])
        bad = np.abs(Lg - ref["y"][i, k]) > ref["tol"][i, k]
        assert not np.any(bad), (f"r{r} k{k + 1}: {bad.sum()} logits off; worst idx "
                                 f"{np.argmax(np.abs(Lg - ref['y'][i, k]) - ref['tol'][i, k])}")
        if qs is not None:
            check_drafted_row_stats(qs[r, k], Lg, ref["L"][i, k], V, T, what=f"q_stats r{r} k{k + 1}")

    def shift(i, r, k):
        return cdf_shift(_f(out["q_logits"][r, k]), ref["rows"][i, k], V, T)

    near, parted, compared, gone = compare_draft_chains(to_np(out["tokens"]), to_np(out["conf"]), ref,
                                                        reqs, check_logits, shift)
    print(f"positions compared={compared} near-boundary draws={near} chains parted={parted}")
    return compared, parted, gone


def test_markov_small_full():
    inp = markov_inputs(R=5, gamma=4, V=2008, rank=64, H=64, rank_e=32, sigma_u=2.0,
                        sigma_f=0.3, seed=91, device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    ref = oracle_chain(inp, range(5), keep=range(5))
    compared, parted, _ = check_chain(inp, out, ref, range(5))
    assert parted <= partings_bound(compared)


def test_markov_smallest_vocabulary():
    """V = 8: one tile of which only 8 of the 128 columns exist, so every
    stage past the first holds no vocabulary column at all."""
    inp = markov_inputs(R=3, gamma=3, V=8, rank=32, H=8, rank_e=8, sigma_u=1.0, sigma_f=0.3, seed=92,
                        device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    ref = oracle_chain(inp, range(3), keep=range(3))
    compared, parted, _ = check_chain(inp, out, ref, range(3))
    assert parted <= partings_bound(compared)


def test_markov_single_request_single_position():
    """R = 1, gamma = 1: one bias launch whose only row block holds one
    request, one select, one confidence; and the full rank (256)."""
    inp = markov_inputs(R=1, gamma=1, V=3000, rank=256, H=8, rank_e=8, sigma_u=1.0, sigma_f=0.1, seed=93,
                        device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    ref = oracle_chain(inp, range(1), keep=range(1))
    compared, parted, _ = check_chain(inp, out, ref, range(1))
    assert parted <= partings_bound(compared)


@pytest.mark.parametrize("rank", [96, 160, 224])
def test_markov_ranks_off_the_powers_of_two(rank):
    """rank = 32 * 3, 5, 7: C rows of 12, 20, 28 sixteen-byte chunks (the LDS
    swizzle groups by the largest power of two dividing that count) and 7,
    9, 11 copies per loader wave and stage; a ragged last tile (V = 3000)."""
    inp = markov_inputs(R=5, gamma=3, V=3000, rank=rank, H=32, rank_e=16, sigma_u=2.0, sigma_f=0.2,
                        seed=96 + rank, device="cuda")
    out = _run(inp)
    ref = oracle_chain(inp, range(5), keep=range(5))
    compared, parted, _ = check_chain(inp, out, ref, range(5))
    assert parted <= partings_bound(compared)


def test_markov_vocab_beyond_1024_tiles():
    """V = 300000: 2344 column tiles, so each select thread combines a run of
    ten tile partials (four of them preloaded) before the walk."""
    inp = markov_inputs(R=3, gamma=2, V=300000, rank=32, H=16, rank_e=8, sigma_u=2.0, sigma_f=0.3,
                        seed=97, device="cuda")
    out = _run(inp)
    ref = oracle_chain(inp, range(3), keep=range(3))
    compared, parted, _ = check_chain(inp, out, ref, range(3))
    assert parted <= partings_bound(compared)


@pytest.mark.parametrize("T", [0.6, 2.0])
def test_markov_temperature(T):
    """Drafting at T != 1: logits divided by T before the draw; the rows'
    (m, Z) reported at that temperature."""
    inp = markov_inputs(R=6, gamma=4, V=3000, rank=64, H=32, rank_e=16, sigma_u=2.0, sigma_f=0.3,
                        seed=95, device="cuda")
    inp["temperature"] = T
    out = _run(inp)
    ref = oracle_chain(inp, range(6), keep=range(6))
    compared, parted, _ = check_chain(inp, out, ref, range(6))
    assert parted <= partings_bound(compared)


def test_markov_whole_block_matches_the_oracle_draft():
    """The oracle's whole-block entry point (markov_draft) on the same inputs:
    tokens equal up to a near-boundary parting, statuses equal."""
    inp = markov_inputs(R=6, gamma=5, V=1000, rank=32, H=16, rank_e=8, sigma_u=1.5,
                        sigma_f=0.5, seed=92, device="cuda")
    out = _run(inp)
    ref = OM.markov_draft(_f(inp["U"]), _f(inp["A"]), _f(inp["Ct"]).transpose(0, 2, 1), to_np(inp["x0"]),
                          _f(inp["h"]), _f(inp["E"]), _f(inp["w"]), 1.0, inp["seed"])
    _, parted, compared, gone = compare_draft_chains(
        to_np(out["tokens"]), to_np(out["conf"]), ref, range(6),
        shift=lambda i, r, k: cdf_shift(_f(out["q_logits"][r, k]), ref["L"][i, k], inp["V"], 1.0))
    assert parted <= partings_bound(compared)
    st = to_np(out["status"])
    for r in range(6):
        if r not in gone:
            assert st[r] == ref["status"][r]


def test_markov_two_row_blocks_and_pos0():
    inp = markov_inputs(R=130, gamma=2, V=1000, rank=32, H=8, rank_e=8, sigma_u=2.0,
                        sigma_f=0.4, seed=93, device="cuda")
    inp["pos0"] = torch.arange(130, dtype=torch.int64, device="cuda") * 7
    out = _run(inp)
    ref = oracle_chain(inp, range(130), keep=(0, 64, 127, 128, 129))
    compared, parted, _ = check_chain(inp, out, ref, range(130))
    assert parted <= partings_bound(compared)


def test_markov_degenerate_anchor_and_rows():
    inp = markov_inputs(R=3, gamma=2, V=512, rank=32, H=8, rank_e=8, seed=94, device="cuda")
    inp["x0"][0] = -1
    inp["U"][1, 0, :] = float("-inf")
    inp["U"][2, 1, 3] = float("nan")
    out = _run(inp)
    st = to_np(out["status"])
    toks = to_np(out["tokens"])
    qs = to_np(out["q_stats"])
    assert st[0] == sdv.SD_ST_BAD_TOKEN
    assert st[1] & sdv.SD_ST_ZERO_Z and toks[1, 0] == -1 and st[1] & sdv.SD_ST_BAD_TOKEN
    assert st[2] & sdv.SD_ST_NONFINITE and toks[2, 1] == -1
    assert qs[1, 0, 0] == -np.inf and qs[1, 0, 1] == 0.0     # an all -inf row reports (-inf, 0)
    assert np.isnan(qs[2, 1, 1])                              # a NaN row: Z is NaN
    ref = oracle_chain(inp, range(3), keep=range(3))
    check_chain(inp, out, ref, [0])                           # no bias, no embedding: still exact


# sixteen requests spread over R = 128 whose logits and (m, Z) are compared
# element by element at every position along the shared history
SAMPLED = (0, 8, 17, 25, 34, 42, 51, 59, 68, 76, 85, 93, 102, 110, 119, 127)


@pytest.fixture(scope="module")
def workload():
    """R=128, gamma=16, V=129280, rank 256: the GPU's block and the oracle's
    chain for every request (logits kept for the sampled requests)."""
    inp = markov_config(device="cuda")
    out = _run(inp)
    ref = oracle_chain(inp, range(inp["R"]), keep=SAMPLED)
    return inp, out, ref


def test_markov_draft_workload_sampled(workload):
    """Logits and (m, Z) on sixteen requests spread over the batch,
    confidences and tokens of every request along the shared histories."""
    inp, out, ref = workload
    assert np.all(to_np(out["status"]) == 0)
    compared, parted, _ = check_chain(inp, out, ref, range(inp["R"]))
    assert parted <= partings_bound(compared)


def test_markov_schedule_and_verify_pipeline(workload):
    """One step of the pipeline at the same sizes: schedule on the drafted
    confidences, verify the drafted rows against target rows (seeded from the
    backbone logits) with the head's (m, Z) handed to the verifier.  The
    oracle runs the same pipeline from the same seeded inputs: its own chain,
    its own schedule, its own verification.  The schedules must agree when no
    chain parted (a parted chain drafts other confidences); verification is
    also run on the oracle's lengths and compared on sampled requests whose
    chains did not part."""
    inp, out, ref = workload
    R, gamma, V = inp["R"], inp["gamma"], inp["V"]
    tgt, sps = markov_targets(inp["U"])
    t0 = torch.arange(R, dtype=torch.int32, device="cuda") * (gamma + 1)
    d0 = torch.arange(R, dtype=torch.int32, device="cuda") * gamma
    drf = out["q_logits"].view(R * gamma, V)

    def verify(ell_dev, lazy=False):
        res = sdv.sd_verify(tgt, t0, drf, d0, out["tokens"], ell_dev, V, 1.0, inp["seed"] + 1, probe=True,
                            stats=True, drf_stats=out["q_stats"], stop_at_rejection=lazy)
        torch.cuda.synchronize()
        return res

    # the GPU pipeline as it runs: structurally valid on every request
    sched = sdv.sd_schedule(out["conf"], sps, OS.EARLY_STOP)
    run = verify(sched["ell"])
    ell_g, n_acc, toks = to_np(sched["ell"]), to_np(run["n_acc"]), to_np(run["tokens"])
    drafted = to_np(out["tokens"])
    assert np.all(to_np(run["status"]) == 0)
    for r in range(R):
        n = n_acc[r]
        assert 0 <= n <= ell_g[r] and np.array_equal(toks[r, :n], drafted[r, :n]) and 0 <= toks[r, n] < V

    compared, parted, gone = check_chain(inp, out, ref, range(R))
    assert parted <= partings_bound(compared)
    ref_s = OS.schedule(ref["conf"].astype(np.float32), to_np(sps), OS.EARLY_STOP)
    if not gone:
        assert np.array_equal(ell_g, ref_s["ell"])
    reqs = [r for r in SAMPLED if r not in gone]
    assert len(reqs) >= 2
    tgt_h = to_np(tgt.view(R, gamma + 1, V)[reqs]).astype(np.float64)
    # the oracle's scheduled lengths, then the whole block (more accept
    # tests), read in one pass and in rounds stopping at the first rejection
    for name, ell, lazy in (("scheduled", ref_s["ell"], False), ("whole block", np.full(R, gamma), False),
                            ("whole block, in rounds", np.full(R, gamma), True)):
        gpu = verify(torch.as_tensor(ell, dtype=torch.int32, device="cuda"), lazy)
        tr0, dr0, tgt_rows, drf_rows = [], [], [], []
        for n, r in enumerate(reqs):
            L = int(ell[r])
            tr0.append(len(tgt_rows))
            tgt_rows.extend(tgt_h[n, :L + 1])
            dr0.append(len(drf_rows))
            drf_rows.extend(ref["rows"][r, j].astype(np.float64) for j in range(L))   # the oracle's own rows
        fn = OV.verify_until_rejection if lazy else OV.verify
        ora = fn(np.array(tgt_rows), np.array(tr0), np.array(drf_rows) if drf_rows else np.zeros((1, V)),
                 np.array(dr0), ref["tokens"][reqs], ell[reqs], V, 1.0, inp["seed"] + 1, req_ids=reqs)
        n_dec, n_near, mism = compare_verify(gpu, ora, reqs)
        print(f"{name}: rows gpu={R + int(ell_g.sum())} oracle={ref_s['B']}; verify decisions={n_dec} "
              f"near-boundary={n_near} diverged={mism}")
        assert mism <= 1
        if lazy:   # the rows read depend on the decisions; those are compared above
            continue
        check_stats(gpu, ora, reqs, ell, gamma, draft=False)
        rs = to_np(gpu["row_stats"])
        for r in reqs:   # the draft slots report the head's (m, Z) of its own rows
            for j in range(int(ell[r])):
                check_drafted_row_stats(rs[r, gamma + 1 + j], _f(out["q_logits"][r, j]), ref["rows"][r, j],
                                        V, 1.0, what=f"draft row r{r} j{j + 1}")
