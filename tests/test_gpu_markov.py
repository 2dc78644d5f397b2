"""GPU parity of sd_markov_draft against the oracle, with teacher forcing.

For every checked (request, position) the oracle is given the GPU's previous
token and computes the exact pre-rounding logits y = U + A_k[x] . C_k (fp64):
the GPU's bf16 logits must be a round-to-nearest of some value within
1e-5 * sum|A_k[x]_i C_k[i, v]| (+ fp32 rounding of the add) of y.  The token
is then re-drawn by the oracle from the GPU's rounded logits and must match
unless near-boundary; the confidence must match within 1e-5 relative.
"""

import numpy as np
import pytest
import torch

import draft_verification_amd as sdv
from oracle import markov as OM
from oracle import schedule as OS
from workloads import markov_inputs, markov_config, markov_targets
from tests.parity_util import (to_np, oracle_verify_subset, compare_verify, check_stats, NEAR,
                               assert_rel)

pytestmark = pytest.mark.gpu


def _run(inp):
    out = sdv.sd_markov_draft(inp["U"], inp["A"], inp["Ct"], inp["x0"], inp["h"], inp["E"], inp["w"],
                              inp["temperature"], inp["seed"], pos0=inp.get("pos0"))
    torch.cuda.synchronize()
    return out


def _bf16_half_ulp(y):
    _, e = np.frexp(y)
    e = np.maximum(e, -125)
    return np.ldexp(0.5, e - 8)


def _teacher_forced_check(inp, out, reqs):
    T, seed = inp["temperature"], inp["seed"]
    toks = to_np(out["tokens"])
    conf = to_np(out["conf"])
    ql = out["q_logits"]
    x0 = to_np(inp["x0"])
    gamma = inp["gamma"]
    H = inp["H"]
    near = 0
    mism = 0
    w = to_np(inp["w"]).astype(np.float64)
    E = inp["E"]
    for k in range(1, gamma + 1):
        A_k = to_np(inp["A"][k - 1]).astype(np.float64)
        C_k = to_np(inp["Ct"][k - 1]).astype(np.float64).T
        for r in reqs:
            xp = int(x0[r]) if k == 1 else int(toks[r, k - 2])
            U = to_np(inp["U"][r, k - 1]).astype(np.float64)[None]
            h = to_np(inp["h"][r, k - 1]).astype(np.float64)[None]
            y, L, _, c, st, _ = OM.markov_step(U, A_k, C_k, [xp], h, to_np(E).astype(np.float64),
                                               w, T, seed, [r], [k])
            Lg = to_np(ql[r, k - 1]).astype(np.float64)
            if 0 <= xp < inp["V"]:
                terms = np.abs(A_k[xp]) @ np.abs(C_k)
            else:
                terms = np.zeros(inp["V"])
            tol = _bf16_half_ulp(y[0]) + 1e-5 * terms + 1e-7 * np.abs(y[0]) + 1e-30
            bad = np.abs(Lg - y[0]) > tol
            assert not np.any(bad), f"r{r} k{k}: {bad.sum()} logits off; worst idx {np.argmax(np.abs(Lg - y[0]) - tol)}"
            assert_rel(conf[r, k - 1], c[0], what=f"conf r{r} k{k}")
            # re-draw from the GPU's rounded logits with the oracle's sampler
            _, _, tok, _, _, dist = OM.markov_step(Lg[None], A_k, np.zeros_like(C_k), [xp], h,
                                                   to_np(E).astype(np.float64), w, T, seed, [r], [k])
            if toks[r, k - 1] != tok[0]:
                assert dist[0] < NEAR, f"r{r} k{k}: gpu token {toks[r, k-1]} vs oracle {tok[0]}"
                mism += 1
            if dist[0] < NEAR:
                near += 1
    return near, mism


def test_markov_small_full():
    inp = markov_inputs(R=5, gamma=4, V=2008, rank=64, H=64, rank_e=32, sigma_u=2.0,
                        sigma_f=0.3, seed=91, device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    near, mism = _teacher_forced_check(inp, out, range(5))
    print(f"near-boundary draws={near} diverged={mism}")
    assert mism <= 1


def test_markov_untied_run_matches_oracle_chain():
    """Without teacher forcing: the oracle's own sequential chain reproduces
    the GPU's tokens unless a near-boundary draw diverged."""
    inp = markov_inputs(R=6, gamma=5, V=1000, rank=32, H=16, rank_e=8, sigma_u=1.5,
                        sigma_f=0.5, seed=92, device="cuda")
    out = _run(inp)
    f = lambda t: to_np(t).astype(np.float64)
    ref = OM.markov_draft(f(inp["U"]), f(inp["A"]), f(inp["Ct"]).transpose(0, 2, 1), to_np(inp["x0"]),
                          f(inp["h"]), f(inp["E"]), f(inp["w"]), 1.0, inp["seed"])
    toks = to_np(out["tokens"])
    for r in range(6):
        if not np.array_equal(toks[r], ref["tokens"][r]):
            k = int(np.argmax(toks[r] != ref["tokens"][r]))
            assert ref["dists"][r, k] < NEAR


def test_markov_two_row_blocks_and_pos0():
    inp = markov_inputs(R=130, gamma=2, V=1000, rank=32, H=8, rank_e=8, sigma_u=2.0,
                        sigma_f=0.4, seed=93, device="cuda")
    inp["pos0"] = torch.arange(130, dtype=torch.int64, device="cuda") * 7
    out = _run(inp)
    # oracle positions include pos0: check by shifting pos in the teacher-forced step
    toks = to_np(out["tokens"])
    pos0 = to_np(inp["pos0"])
    for r in (0, 64, 127, 128, 129):
        for k in (1, 2):
            xp = int(to_np(inp["x0"])[r]) if k == 1 else int(toks[r, 0])
            A_k = to_np(inp["A"][k - 1]).astype(np.float64)
            Lg = to_np(out["q_logits"][r, k - 1]).astype(np.float64)
            _, _, tok, _, _, dist = OM.markov_step(
                Lg[None], A_k, np.zeros((32, 1000)), [xp], to_np(inp["h"][r, k - 1]).astype(np.float64)[None],
                to_np(inp["E"]).astype(np.float64), to_np(inp["w"]).astype(np.float64), 1.0,
                inp["seed"], [r], [int(pos0[r]) + k])
            assert toks[r, k - 1] == tok[0] or dist[0] < NEAR


def test_markov_degenerate_anchor_and_rows():
    inp = markov_inputs(R=3, gamma=2, V=512, rank=32, H=8, rank_e=8, seed=94, device="cuda")
    inp["x0"][0] = -1
    inp["U"][1, 0, :] = float("-inf")
    inp["U"][2, 1, 3] = float("nan")
    out = _run(inp)
    st = to_np(out["status"])
    toks = to_np(out["tokens"])
    assert st[0] == sdv.SD_ST_BAD_TOKEN
    assert st[1] & sdv.SD_ST_ZERO_Z and toks[1, 0] == -1 and st[1] & sdv.SD_ST_BAD_TOKEN
    assert st[2] & sdv.SD_ST_NONFINITE and toks[2, 1] == -1


def test_markov_draft_workload_sampled():
    """R=128, gamma=16, V=129280, rank 256: checked on sampled requests for all
    16 positions; then scheduled and verified end to end."""
    inp = markov_config(device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    near, mism = _teacher_forced_check(inp, out, [0, 77, 127])
    print(f"near-boundary draws={near} diverged={mism} of {16 * 3}")
    assert mism <= 1
    # confidences of every (r, k) (cheap): oracle with the GPU's previous tokens
    toks = to_np(out["tokens"])
    x0 = to_np(inp["x0"])
    prev = np.concatenate([x0[:, None], toks[:, :-1]], axis=1)
    h = to_np(inp["h"]).astype(np.float64)
    E = to_np(inp["E"]).astype(np.float64)
    w = to_np(inp["w"]).astype(np.float64)
    z = h @ w[:inp["H"]] + E[prev] @ w[inp["H"]:]
    assert_rel(to_np(out["conf"]), OM.sigmoid(z), what="conf")

    # end to end: targets from the drafted rows, schedule, verify
    R, gamma, V = inp["R"], inp["gamma"], inp["V"]
    tgt, sps = markov_targets(out["q_logits"])
    vin = dict(R=R, gmax=gamma, V=V, temperature=1.0, seed=inp["seed"] + 1, pos0=None, tgt=tgt,
               drf=out["q_logits"].view(R * gamma, V),
               tgt_row0=torch.arange(R, dtype=torch.int32, device="cuda") * (gamma + 1),
               drf_row0=torch.arange(R, dtype=torch.int32, device="cuda") * gamma,
               draft_tokens=out["tokens"])
    sched = sdv.sd_schedule(out["conf"], sps, OS.EARLY_STOP)
    ref_s = OS.schedule(to_np(out["conf"]), to_np(sps), OS.EARLY_STOP)
    assert np.array_equal(to_np(sched["ell"]), ref_s["ell"])
    gpu = sdv.sd_verify(vin["tgt"], vin["tgt_row0"], vin["drf"], vin["drf_row0"], vin["draft_tokens"],
                        sched["ell"], V, 1.0, vin["seed"], probe=True, stats=True)
    torch.cuda.synchronize()
    reqs = [0, 5, 77, 127]
    ora = oracle_verify_subset(vin, reqs, ref_s["ell"])
    n_dec, n_near, mism = compare_verify(gpu, ora, reqs)
    print(f"verify decisions={n_dec} near-boundary={n_near} diverged={mism}")
    assert mism <= 1
    check_stats(gpu, ora, reqs, ref_s["ell"], gamma)
