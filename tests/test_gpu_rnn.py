"""GPU parity of sd_rnn_draft against the oracle.

As for the Markov head, every drafted token is a draw whose history is the
GPU's own earlier tokens, and several tokens are correct where a draw is
near-boundary; so each position is checked given the drafted history: the
oracle recomputes the recurrent state along that history and the exact logits
y = U + s . C (fp64).  The GPU's bf16 logits must be a round-to-nearest of a
value within 1e-5 * sum|s_i C_i| + 1e-5 * sum|C_i| + 1e-7 * |y| of y (the
middle term bounds the fp32 state's error, the two-term bf16 split included).
The token is re-drawn by the oracle from the GPU's rounded logits and must
match unless near-boundary; the confidence must match within 1e-5 relative.
Without teacher forcing, the oracle's own chain must reproduce the GPU's
tokens up to the first near-boundary draw.
"""

import numpy as np
import pytest
import torch

import draft_verification_amd as sdv
from oracle import markov as OM
from oracle import rnn as ON
from workloads import rnn_config, rnn_inputs
from tests.parity_util import to_np, NEAR, assert_rel

pytestmark = pytest.mark.gpu


def _run(inp):
    out = sdv.sd_rnn_draft(inp["U"], inp["W"], inp["Es"], inp["Ct"], inp["x0"], inp["h"], inp["E"],
                           inp["w"], inp["temperature"], inp["seed"], pos0=inp.get("pos0"))
    torch.cuda.synchronize()
    return out


def _bf16_half_ulp(y):
    _, e = np.frexp(y)
    e = np.maximum(e, -125)
    return np.ldexp(0.5, e - 8)


def _f(t):
    return to_np(t).astype(np.float64)


def _teacher_forced_check(inp, out, reqs):
    T, seed, V = inp["temperature"], inp["seed"], inp["V"]
    toks = to_np(out["tokens"])
    conf = to_np(out["conf"])
    W, Es, C = _f(inp["W"]), _f(inp["Es"]), _f(inp["Ct"]).T
    E, w = _f(inp["E"]), _f(inp["w"])
    absC = np.abs(C)
    x0 = to_np(inp["x0"])
    pos0 = np.zeros(inp["R"], np.int64) if inp.get("pos0") is None else to_np(inp["pos0"])
    near = mism = 0
    for r in reqs:
        s = np.zeros((1, W.shape[0]))
        for k in range(1, inp["gamma"] + 1):
            xp = int(x0[r]) if k == 1 else int(toks[r, k - 2])
            U = _f(inp["U"][r, k - 1])[None]
            h = _f(inp["h"][r, k - 1])[None]
            s, y, L, _, c, _, _ = ON.rnn_step(U, W, Es, C, s, [xp], h, E, w, T, seed, [r],
                                              [int(pos0[r]) + k])
            Lg = _f(out["q_logits"][r, k - 1])
            tol = (_bf16_half_ulp(y[0]) + 1e-5 * (np.abs(s[0]) @ absC) + 1e-5 * absC.sum(axis=0)
                   + 1e-7 * np.abs(y[0]) + 1e-30)
            bad = np.abs(Lg - y[0]) > tol
            assert not np.any(bad), f"r{r} k{k}: {bad.sum()} logits off"
            assert_rel(conf[r, k - 1], c[0], what=f"conf r{r} k{k}")
            # re-draw from the GPU's rounded logits with the oracle's sampler
            _, tok, _, _, dist = OM.draw_position(Lg[None], [xp], h, E, w, T, seed, [r],
                                                  [int(pos0[r]) + k], np.zeros(1, np.int32))
            if toks[r, k - 1] != tok[0]:
                assert dist[0] < NEAR, f"r{r} k{k}: gpu token {toks[r, k - 1]} vs oracle {tok[0]}"
                mism += 1
            if dist[0] < NEAR:
                near += 1
    return near, mism


def test_rnn_small_full():
    inp = rnn_inputs(R=5, gamma=4, V=2008, d=64, H=64, rank_e=32, sigma_c=0.3, seed=95, device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    near, mism = _teacher_forced_check(inp, out, range(5))
    print(f"near-boundary draws={near} diverged={mism}")
    assert mism <= 1


@pytest.mark.parametrize("d", [32, 96, 128])
def test_rnn_state_sizes_and_positions(d):
    inp = rnn_inputs(R=9, gamma=6, V=1000, d=d, H=16, rank_e=8, sigma_c=0.4, seed=96 + d, device="cuda")
    inp["pos0"] = torch.arange(9, dtype=torch.int64, device="cuda") * 31 + 5
    out = _run(inp)
    near, mism = _teacher_forced_check(inp, out, range(9))
    assert mism <= 1


def test_rnn_untied_run_matches_oracle_chain():
    inp = rnn_inputs(R=6, gamma=6, V=1000, d=64, H=16, rank_e=8, sigma_u=1.5, sigma_c=0.5, seed=97,
                     device="cuda")
    out = _run(inp)
    ref = ON.rnn_draft(_f(inp["U"]), _f(inp["W"]), _f(inp["Es"]), _f(inp["Ct"]).T, to_np(inp["x0"]),
                       _f(inp["h"]), _f(inp["E"]), _f(inp["w"]), 1.0, inp["seed"])
    toks = to_np(out["tokens"])
    for r in range(6):
        if not np.array_equal(toks[r], ref["tokens"][r]):
            k = int(np.argmax(toks[r] != ref["tokens"][r]))
            assert ref["dists"][r, k] < NEAR


def test_rnn_more_than_one_row_block():
    inp = rnn_inputs(R=130, gamma=2, V=1000, d=32, H=8, rank_e=8, sigma_c=0.4, seed=98, device="cuda")
    out = _run(inp)
    near, mism = _teacher_forced_check(inp, out, [0, 64, 127, 128, 129])
    assert mism <= 1


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
    # the state keeps going without an embedding term: later positions still check out
    near, mism = _teacher_forced_check(inp, out, [0])
    assert mism <= 1


def test_rnn_draft_workload_sampled():
    """R=128, gamma=16, V=129280, d=128: sampled requests for all 16 positions,
    confidences of every (r, k)."""
    inp = rnn_config(device="cuda")
    out = _run(inp)
    assert np.all(to_np(out["status"]) == 0)
    near, mism = _teacher_forced_check(inp, out, [0, 77, 127])
    print(f"near-boundary draws={near} diverged={mism} of {16 * 3}")
    assert mism <= 1
    toks = to_np(out["tokens"])
    prev = np.concatenate([to_np(inp["x0"])[:, None], toks[:, :-1]], axis=1)
    z = _f(inp["h"]) @ _f(inp["w"])[:inp["H"]] + _f(inp["E"])[prev] @ _f(inp["w"])[inp["H"]:]
    assert_rel(to_np(out["conf"]), OM.sigmoid(z), what="conf")


def test_rnn_host_errors():
    inp = rnn_inputs(R=2, gamma=2, V=64, d=32, H=8, rank_e=8, seed=100, device="cuda")
    W48 = torch.zeros((48, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdv.SdvError):
        sdv.sd_rnn_draft(inp["U"], W48, inp["Es"], inp["Ct"], inp["x0"], inp["h"], inp["E"], inp["w"])
    W160 = torch.zeros((160, 160), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_rnn_draft(inp["U"], W160, inp["Es"], inp["Ct"], inp["x0"], inp["h"], inp["E"], inp["w"])
    assert e.value.code == -3
