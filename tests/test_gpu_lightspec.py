"""GPU parity of the two-stage budget planner (sd_lightspec_update,
sd_lightspec_plan) against the oracle: the EMA state, the planning
confidences, both stages' choices and Phi must be bit-identical on the same
inputs."""

import numpy as np
import pytest
import torch

import draft_verification_amd as sdv
from oracle import lightspec as OL
from oracle.verify import ST_NONFINITE, ST_ZERO_Z
from workloads import verify_config, sps_table
from tests.parity_util import oracle_verify_subset, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _t(x, dtype):
    return torch.as_tensor(np.asarray(x), dtype=dtype).to(DEV).contiguous()


def _update_case(g, R, G):
    alpha = g.uniform(0.0, 1.0, (R, G)).astype(np.float32)
    ell = g.integers(-1, G + 2, R).astype(np.int32)          # out-of-range lengths are clamped
    status = np.zeros(R, np.int32)
    status[g.integers(0, R, max(1, R // 10))] = g.choice([ST_NONFINITE, ST_ZERO_Z, 1, 8])
    return alpha, ell, status


@pytest.mark.parametrize("R,G", [(1, 1), (7, 5), (256, 11), (512, 16), (40, 255)])
def test_update_matches_oracle_over_several_steps(R, G):
    g = np.random.default_rng(R * 1000 + G)
    ema_o = g.uniform(0.0, 1.0, G)
    cnt_o = np.zeros(G, np.int64)
    cnt_o[g.integers(0, G, max(1, G // 3))] = 5            # some positions already observed
    ema_g, cnt_g = _t(ema_o, torch.float64), _t(cnt_o, torch.int64)
    for step, lam in enumerate((0.1, 0.5, 1.0, 0.0, 0.05)):
        alpha, ell, status = _update_case(g, R, G)
        sdv.sd_lightspec_update(_t(alpha, torch.float32), _t(ell, torch.int32),
                                _t(status, torch.int32), lam, ema_g, cnt_g)
        ema_o, cnt_o = OL.ema_update(alpha, ell, status, lam, ema_o, cnt_o)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(ema_g), ema_o), step
        assert np.array_equal(to_np(cnt_g), cnt_o), step


def _plan_both(ema, cnt, d_prev, sps, cost):
    got = sdv.sd_lightspec_plan(_t(ema, torch.float64), _t(cnt, torch.int64), _t(d_prev, torch.int32),
                                _t(sps, torch.float32), _t(cost, torch.float32))
    torch.cuda.synchronize()
    got = {k: to_np(v) for k, v in got.items()}
    ref = OL.plan(ema, cnt, d_prev, sps, cost)
    assert np.array_equal(got["conf"], ref["conf"])
    assert np.array_equal(got["ell"], ref["ell"])
    assert int(got["batch"][0]) == ref["B"] and int(got["n_sel"][0]) == ref["n_sel"]
    assert float(got["theta"][0]) == ref["theta"]
    assert np.array_equal(got["phi"], ref["phi"])
    assert int(got["d_next"][0]) == ref["d_next"] and int(got["b_next"][0]) == ref["b_next"]
    return got, ref


@pytest.mark.parametrize("R,G", [(1, 1), (3, 3), (64, 8), (256, 11), (1024, 16), (16, 255)])
def test_plan_matches_oracle(R, G):
    g = np.random.default_rng(7 * R + G)
    for case in range(3):
        ema = np.sort(g.uniform(0.2, 1.0, G))[::-1].copy()
        cnt = (g.uniform(size=G) < 0.6).astype(np.int64) * g.integers(1, 50, G)
        if case == 1:
            cnt[:] = 0                                    # nothing observed: the prior
        if case == 2 and G > 2:
            ema[1] = 1.0                                  # equal survivals at positions 1, 2
            cnt[:] = 1
        d_prev = g.integers(0, G + 1, R).astype(np.int32)
        Bs = np.arange(1, R * (G + 1) + 1, dtype=np.float64)
        sps = (1.0 / (0.002 * Bs ** 0.5 + 0.01) * (1 + 0.05 * ((Bs - 1) % 64 / 32 - 1))).astype(np.float32)
        cost = (0.004 * np.arange(1, G + 1) + g.uniform(0, 0.002, G)).astype(np.float32)
        _plan_both(ema, cnt, d_prev, sps, cost)


def test_plan_headline_table_and_uniform_drafts():
    """R=256 requests, gamma=11, the headline workload's throughput table."""
    inp = verify_config("headline", device="cpu", V=64)
    R, G = inp["R"], inp["gmax"]
    sps = inp["sps"].numpy()
    ema = np.linspace(0.9, 0.45, G)
    cnt = np.ones(G, np.int64)
    cost = (0.0008 * np.arange(1, G + 1)).astype(np.float32) * float(np.median(1.0 / sps))
    got, ref = _plan_both(ema, cnt, np.full(R, G, np.int32), sps, cost)
    assert 1 <= ref["d_next"] <= G


def test_closed_loop_after_verification():
    """mid workload: verify with acceptance rates on the GPU, fold them into
    the EMA, plan.  The oracle runs the same loop from its own acceptance
    rates; the EMA agrees to the acceptance rates' tolerance."""
    inp = verify_config("mid", device=DEV)
    R, G = inp["R"], inp["gmax"]
    ell = torch.full((R,), G, dtype=torch.int32, device=DEV)
    out = sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"], inp["draft_tokens"],
                        ell, inp["V"], inp["temperature"], inp["seed"], alpha=True)
    ema, cnt = torch.full((G,), 0.5, dtype=torch.float64, device=DEV), torch.zeros(G, dtype=torch.int64,
                                                                                       device=DEV)
    sdv.sd_lightspec_update(out["alpha"], ell, out["status"], 0.2, ema, cnt)
    plan = sdv.sd_lightspec_plan(ema, cnt, ell, inp["sps"], torch.full((G,), 1e-3, device=DEV))
    torch.cuda.synchronize()
    ora = oracle_verify_subset(inp, list(range(R)), to_np(ell))
    ema_o, cnt_o = OL.ema_update(ora["alpha"], to_np(ell), ora["status"], 0.2, np.full(G, 0.5),
                                 np.zeros(G, np.int64))
    assert np.array_equal(to_np(cnt), cnt_o)
    assert np.allclose(to_np(ema), ema_o, rtol=0, atol=1e-7)
    assert np.allclose(to_np(plan["conf"]), OL.conf_hat(ema_o, cnt_o), rtol=0, atol=2e-7)
    assert 1 <= int(plan["d_next"].item()) <= G
