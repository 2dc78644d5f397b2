"""GPU parity of sd_rnn_draft against the oracle.

As for the Markov head, the oracle runs its own chain (recurrent state
included) from the same seeded inputs; no GPU output enters it.  Along the
history the two chains share, each GPU bf16 logit must be a round-to-nearest
of a value within 1e-5 * sum|s_i C_i| + 1e-5 * sum|C_i| + 1e-7 * |y| of the
oracle's exact y = U + s . C (fp64; the middle term bounds the fp32 state's
error; its three bf16 terms carry it exactly); the confidence and the row's
(m, Z) must match within 1e-5 relative; tokens must be equal except where
the oracle's draw is near-boundary, where the chains may part and the rest of
that request is not compared.
"""

import numpy as np
import pytest
import torch

import draft_verification_amd as sdv
from oracle import rnn as ON
from workloads import rnn_config, rnn_inputs
from tests.parity_util import (to_np, compare_draft_chains, bf16_half_ulp, partings_bound,
                               check_drafted_row_stats, cdf_shift)

pytestmark = pytest.mark.gpu


def _run(inp, stats=True):
    out = sdv.sd_rnn_draft(inp["U"], inp["W"], inp["Es"], inp["Ct"], inp["x0"], inp["h"], inp["E"],
                           inp["w"], inp["temperature"], inp["seed"], pos0=inp.get("pos0"), stats=stats)
    torch.cuda.synchronize()
    return out


def _f(t):
    return to_np(t).astype(np.float64)


def oracle_chain(inp, reqs, keep=()):
    """The oracle's RNN chain for requests `reqs`, from the seeded inputs
    alone; for the requests in `keep` it keeps, per position, the exact
    logits y, the rounded L and the logits' tolerance."""
    T, seed, V, gamma = inp["temperature"], inp["seed"], inp["V"], inp["gamma"]
    reqs = [int(r) for r in reqs]
    n = len(reqs)
    W, Es, C = _f(inp["W"]), _f(inp["Es"]), _f(inp["Ct"]).T
    E, w = _f(inp["E"]), _f(inp["w"])
    absC = np.abs(C)
    colC = absC.sum(axis=0)
    idx = torch.as_tensor(reqs, dtype=torch.long, device=inp["U"].device)
    U = inp["U"].index_select(0, idx)
    h = inp["h"].index_select(0, idx)
    x_prev = to_np(inp["x0"])[reqs].astype(np.int64)
    pos0 = (np.zeros(n, np.int64) if inp.get("pos0") is None
            else to_np(inp["pos0"])[reqs].astype(np.int64))
    kept = [i for i, r in enumerate(reqs) if r in set(keep)]
    ref = dict(tokens=np.zeros((n, gamma), np.int64), conf=np.zeros((n, gamma)),
               dists=np.zeros((n, gamma)), status=np.zeros(n, np.int32), y={}, L={}, tol={},
               rows=np.zeros((n, gamma, V), np.float32))
    s = np.zeros((n, W.shape[0]))
    for k in range(1, gamma + 1):
        s, y, L, tok, c, st, d = ON.rnn_step(_f(U[:, k - 1]), W, Es, C, s, x_prev, _f(h[:, k - 1]), E, w,
                                             T, seed, reqs, pos0 + k)
        for i in kept:
            ref["y"][i, k - 1] = y[i]
            ref["L"][i, k - 1] = L[i]
            ref["tol"][i, k - 1] = (bf16_half_ulp(y[i]) + 1e-5 * (np.abs(s[i]) @ absC) + 1e-5 * colC
                                    + 1e-7 * np.abs(y[i]) + 1e-30)
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
    qs = to_np(out["q_stats"]) if out.get("q_stats") is not None else None

    def check_logits(i, r, k):
        if (i, k) not in ref["y"]:
            return
        Lg = _f(out["q_logits"][r, k])
        bad = np.abs(Lg - ref["y"][i, k]) > ref["tol"][i, k]
        assert not np.any(bad), f"r{r} k{k + 1}: {bad.sum()} logits off"
        if qs is not None:
            check_drafted_row_stats(qs[r, k], Lg, ref["L"][i, k], V, T, what=f"q_stats r{r} k{k + 1}")

    def shift(i, r, k):
        return cdf_shift(_f(out["q_logits"][r, k]), ref["rows"][i, k], V, T)

    near, parted, compared, gone = compare_draft_chains(to_np(out["tokens"]), to_np(out["conf"]), ref,
                                                        reqs, check_logits, shift)
    print(f"positions compared={compared} near-boundary draws={near} chains parted={parted}")
    return compared, parted, gone


def test_rnn_small_full():
    inp = rnn_inputs(R=5, gamma=4, V=2008, d=64, H=64, rank_e=32, sigma_c=0.3, seed=95, device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    ref = oracle_chain(inp, range(5), keep=range(5))
    compared, parted, _ = check_chain(inp, out, ref, range(5))
    assert parted <= partings_bound(compared)


def test_rnn_smallest_vocabulary():
    """V = 8 and d = 32: one vocabulary tile with 8 live columns."""
    inp = rnn_inputs(R=3, gamma=3, V=8, d=32, H=8, rank_e=8, sigma_c=0.3, seed=96, device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    ref = oracle_chain(inp, range(3), keep=range(3))
    compared, parted, _ = check_chain(inp, out, ref, range(3))
    assert parted <= partings_bound(compared)


def test_rnn_single_request_single_position():
    """R = 1, gamma = 1: the state is initialised and never advanced."""
    inp = rnn_inputs(R=1, gamma=1, V=3000, d=64, H=8, rank_e=8, sigma_c=0.3, seed=97, device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    ref = oracle_chain(inp, range(1), keep=range(1))
    compared, parted, _ = check_chain(inp, out, ref, range(1))
    assert parted <= partings_bound(compared)


@pytest.mark.parametrize("d", [32, 96, 128])
def test_rnn_state_sizes_and_positions(d):
    inp = rnn_inputs(R=9, gamma=6, V=1000, d=d, H=16, rank_e=8, sigma_c=0.4, seed=96 + d, device="cuda")
    inp["pos0"] = torch.arange(9, dtype=torch.int64, device="cuda") * 31 + 5
    out = _run(inp)
    ref = oracle_chain(inp, range(9), keep=range(9))
    compared, parted, _ = check_chain(inp, out, ref, range(9))
    assert parted <= partings_bound(compared)


@pytest.mark.parametrize("T", [0.6, 2.0])
def test_rnn_temperature(T):
    """Drafting at T != 1, as for the Markov head."""
    inp = rnn_inputs(R=6, gamma=4, V=3000, d=64, H=32, rank_e=16, sigma_c=0.3, seed=101, device="cuda")
    inp["temperature"] = T
    out = _run(inp)
    ref = oracle_chain(inp, range(6), keep=range(6))
    compared, parted, _ = check_chain(inp, out, ref, range(6))
    assert parted <= partings_bound(compared)


def test_rnn_whole_block_matches_the_oracle_draft():
    """The oracle's whole-block entry point (rnn_draft) on the same inputs:
    tokens equal up to a near-boundary parting, statuses equal."""
    inp = rnn_inputs(R=6, gamma=6, V=1000, d=64, H=16, rank_e=8, sigma_u=1.5, sigma_c=0.5, seed=97,
                     device="cuda")
    out = _run(inp)
    ref = ON.rnn_draft(_f(inp["U"]), _f(inp["W"]), _f(inp["Es"]), _f(inp["Ct"]).T, to_np(inp["x0"]),
                       _f(inp["h"]), _f(inp["E"]), _f(inp["w"]), 1.0, inp["seed"])
    _, parted, compared, gone = compare_draft_chains(
        to_np(out["tokens"]), to_np(out["conf"]), ref, range(6),
        shift=lambda i, r, k: cdf_shift(_f(out["q_logits"][r, k]), ref["L"][i, k], inp["V"], 1.0))
    assert parted <= partings_bound(compared)
    st = to_np(out["status"])
    for r in range(6):
        if r not in gone:
            assert st[r] == ref["status"][r]


def test_rnn_more_than_one_row_block():
    inp = rnn_inputs(R=130, gamma=2, V=1000, d=32, H=8, rank_e=8, sigma_c=0.4, seed=98, device="cuda")
    out = _run(inp)
    ref = oracle_chain(inp, range(130), keep=(0, 64, 127, 128, 129))
    compared, parted, _ = check_chain(inp, out, ref, range(130))
    assert parted <= partings_bound(compared)


def test_rnn_degenerate_anchor_and_rows():
    inp = rnn_inputs(R=3, gamma=3, V=512, d=32, H=8, rank_e=8, seed=99, device="cuda")
    inp["x0"][0] = -1
    inp["U"][1, 0, :] = float("-inf")
    inp["U"][2, 1, 3] = float("nan")
    out = _run(inp)
    st = to_np(out["status"])
    toks = to_np(out["tokens"])
    assert st[0] == sdv.SD_ST_BAD_TOKEN
    assert st[1] & sdv.SD_ST_ZERO_Z and toks[1, 0] == -1 and st[1] & sdv.SD_ST_BAD_TOKEN
    assert st[2] & sdv.SD_ST_NONFINITE and toks[2, 1] == -1
    # the state keeps going without an embedding term: request 0 still checks out
    ref = oracle_chain(inp, range(3), keep=range(3))
    compared, parted, _ = check_chain(inp, out, ref, [0])
    assert parted <= partings_bound(compared)


def test_rnn_draft_workload_sampled():
    """R=128, gamma=16, V=129280, d=128: the oracle's chain for every request;
    logits and (m, Z) on sixteen requests spread over the batch, confidences
    and tokens everywhere along the shared histories."""
    inp = rnn_config(device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    keep = (0, 8, 17, 25, 34, 42, 51, 59, 68, 76, 85, 93, 102, 110, 119, 127)   # spread over R = 128
    ref = oracle_chain(inp, range(inp["R"]), keep=keep)
    compared, parted, _ = check_chain(inp, out, ref, range(inp["R"]))
    assert parted <= partings_bound(compared)


def test_rnn_host_errors():
    inp = rnn_inputs(R=2, gamma=2, V=64, d=32, H=8, rank_e=8, seed=100, device="cuda")
    W48 = torch.zeros((48, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdv.SdvError):
        sdv.sd_rnn_draft(inp["U"], W48, inp["Es"], inp["Ct"], inp["x0"], inp["h"], inp["E"], inp["w"])
    W160 = torch.zeros((160, 160), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_rnn_draft(inp["U"], W160, inp["Es"], inp["Ct"], inp["x0"], inp["h"], inp["E"], inp["w"])
    assert e.value.code == -3
