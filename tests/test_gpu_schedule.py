"""GPU parity of sd_schedule against the oracle: survival, l_r, B, n*, Theta
must all be bit-identical."""

import numpy as np
import pytest
import torch

import draft_verification_amd as sdv
from oracle import schedule as OS
from workloads import verify_config, sps_table

pytestmark = pytest.mark.gpu

MODES = [OS.EARLY_STOP, OS.GLOBAL_ARGMAX]


def _run(conf, sps, mode, gamma_r=None, cap=None, threshold=0.0, sts=None):
    dev = "cuda"
    c = torch.as_tensor(conf, dtype=torch.float32).to(dev).contiguous()
    s = torch.as_tensor(sps, dtype=torch.float32).to(dev)
    g = None if gamma_r is None else torch.as_tensor(gamma_r, dtype=torch.int32).to(dev)
    k = None if cap is None else torch.tensor([int(cap)], dtype=torch.int32, device=dev)
    t = None if sts is None else torch.as_tensor(sts, dtype=torch.float32).to(dev)
    out = sdv.sd_schedule(c, s, mode, gamma_r=g, cap_k=k, threshold=threshold, sts_temp=t)
    torch.cuda.synchronize()
    return {k2: (v.cpu().numpy() if v is not None else None) for k2, v in out.items()}


def _check(conf, sps, mode, gamma_r=None, cap=None, threshold=0.0, sts=None):
    conf = np.asarray(conf, np.float32)
    got = _run(conf, sps, mode, gamma_r, cap, threshold, sts)
    ref = OS.schedule(conf, sps, mode, gamma_r, cap_k=cap, threshold=threshold,
                      sts_temp=None if sts is None else np.asarray(sts, np.float32))
    assert np.array_equal(got["ell"], ref["ell"]), (got["ell"], ref["ell"])
    assert int(got["batch"][0]) == ref["B"]
    assert int(got["n_sel"][0]) == ref["n_sel"]
    assert float(got["theta"][0]) == ref["theta"]
    assert np.array_equal(got["surv"], ref["surv"])
    return ref


@pytest.mark.parametrize("name", ["tiny", "mid", "headline"])
@pytest.mark.parametrize("mode", MODES)
def test_schedule_workloads(name, mode):
    inp = verify_config(name, device="cpu", V=64)  # only conf and sps are used
    _check(inp["conf"].numpy(), inp["sps"].numpy(), mode)


@pytest.mark.parametrize("levels", [None, (0.25, 0.5, 0.75, 1.0)])
def test_schedule_random_cases(levels):
    g = np.random.default_rng(11 if levels is None else 12)
    for case in range(60):
        R = int(g.integers(1, 48))
        gmax = int(g.integers(1, 17))
        if levels is None:
            conf = (1 / (1 + np.exp(-g.normal(1.0, 1.5, (R, gmax))))).astype(np.float32)
        else:
            conf = g.choice(np.array(levels, np.float32), (R, gmax))
        gam = g.integers(0, gmax + 1, R).astype(np.int32)
        Bs = np.arange(1, R * (gmax + 1) + 1)
        sps = (Bs / (1 + Bs / g.uniform(4, 64)) * (1 + 0.1 * (((Bs - 1) % 8) / 4.0 - 1))).astype(np.float32)
        for mode in MODES:
            _check(conf, sps, mode, gam)
        _check(conf, sps, OS.CAPPED_TOPK, gam, cap=int(g.integers(0, R * gmax + 3)))


def test_schedule_async_chain_on_device():
    """Ragged async step: K from the previous confidences (global argmax), then
    exactly K candidates by the current ones, chained through device memory."""
    inp = verify_config("ragged", device="cpu", V=64)
    conf, prev, sps, gam = inp["conf"], inp["conf_prev"], inp["sps"], inp["gamma_r"]
    dev = "cuda"
    first = sdv.sd_schedule(prev.to(dev), sps.to(dev), OS.GLOBAL_ARGMAX, gamma_r=gam.to(dev))
    second = sdv.sd_schedule(conf.to(dev), sps.to(dev), OS.CAPPED_TOPK, gamma_r=gam.to(dev),
                             cap_k=first["n_sel"])
    torch.cuda.synchronize()
    ref = OS.async_schedule(conf.numpy(), prev.numpy(), sps.numpy(), gam.numpy())
    assert int(first["n_sel"].item()) == ref["cap_k"]
    assert np.array_equal(second["ell"].cpu().numpy(), ref["ell"])
    assert int(second["batch"].item()) == ref["B"]
    assert float(second["theta"].item()) == ref["theta"]


@pytest.mark.parametrize("R,gmax", [(64, 16), (41, 25), (128, 16), (683, 3), (256, 16), (241, 17)])
def test_schedule_sizes_around_the_select_layouts(R, gmax):
    """R * gmax = 1024, 1025, 2048, 2049, 4096, 4097: the selection holds 1, 2,
    4 or 8 sorted positions per thread; ties and ragged lengths included."""
    g = np.random.default_rng(R * 100 + gmax)
    for levels in (None, (0.25, 0.5, 0.75, 1.0)):
        if levels is None:
            conf = (1 / (1 + np.exp(-g.normal(1.0, 1.5, (R, gmax))))).astype(np.float32)
        else:
            conf = g.choice(np.array(levels, np.float32), (R, gmax))
        gam = g.integers(0, gmax + 1, R).astype(np.int32)
        sps = sps_table(R * (gmax + 1), 256, 0.08, 64).numpy()
        for mode in MODES:
            _check(conf, sps, mode, gam)
            _check(conf, sps, mode)
        _check(conf, sps, OS.CAPPED_TOPK, gam, cap=int(g.integers(0, R * gmax + 3)))
        _check(conf, sps, OS.THRESHOLD, gam, threshold=0.3)


@pytest.mark.parametrize("R,gmax", [(1024, 1), (1025, 1), (4, 255), (1, 255), (5, 205), (33, 31)])
def test_schedule_long_chains_and_single_drafts(R, gmax):
    """The longest chains (gamma_max = 255, 205) next to wide batches of
    single drafts, around one candidate per selection thread (1024, 1025),
    with ragged lengths, tied survivals and per-position temperatures."""
    g = np.random.default_rng(R * 1000 + gmax)
    conf = (1 / (1 + np.exp(-g.normal(2.0, 1.5, (R, gmax))))).astype(np.float32)
    conf[:, ::3] = np.float32(0.75)                  # repeated values: tied survivals
    gam = g.integers(0, gmax + 1, R).astype(np.int32)
    sts = (0.5 + g.random(gmax)).astype(np.float32)
    sps = sps_table(R * (gmax + 1), 256, 0.08, 64).numpy()
    for mode in MODES:
        _check(conf, sps, mode, gam)
        _check(conf, sps, mode, sts=sts)
    _check(conf, sps, OS.CAPPED_TOPK, gam, cap=int(g.integers(0, R * gmax + 3)), sts=sts)
    _check(conf, sps, OS.THRESHOLD, gam, threshold=0.3)


def test_schedule_maximum_slots_and_subnormal_survival():
    g = np.random.default_rng(13)
    R, gmax = 1024, 16                          # R * gmax = 16384, the limit
    conf = (1 / (1 + np.exp(-g.normal(0.0, 3.0, (R, gmax))))).astype(np.float32)
    conf[:8] = np.float32(0.004)                # survivals reach the fp32 subnormal range
    sps = sps_table(R * (gmax + 1), 256, 0.08, 64).numpy()
    for mode in MODES:
        _check(conf, sps, mode)
    _check(conf, sps, OS.CAPPED_TOPK, cap=R * gmax - 3)


def test_schedule_degenerate_sizes():
    sps = np.ones(64, np.float32)
    got = _run(np.zeros((5, 0), np.float32), sps, OS.EARLY_STOP)
    assert np.all(got["ell"] == 0) and int(got["batch"][0]) == 5 and float(got["theta"][0]) == 0.0
    conf = np.zeros((3, 4), np.float32)           # zero confidence: Theta stays 0
    _check(conf, sps, OS.EARLY_STOP)
    _check(conf, sps, OS.GLOBAL_ARGMAX)
    _check(np.ones((3, 4), np.float32), sps, OS.EARLY_STOP)


def test_schedule_host_errors():
    dev = "cuda"
    c = torch.rand((4, 4), device=dev)
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_schedule(c, torch.ones(10, device=dev), OS.EARLY_STOP)   # table < 20
    assert e.value.code == -2
    with pytest.raises(sdv.SdvError):
        sdv.sd_schedule(c, torch.ones(20, device=dev), 7)
    with pytest.raises(sdv.SdvError):
        sdv.sd_schedule(c, torch.ones(20, device=dev), OS.CAPPED_TOPK)  # no cap_k


@pytest.mark.parametrize("name", ["tiny", "mid", "headline"])
def test_schedule_threshold_mode(name):
    inp = verify_config(name, device="cpu", V=64)
    conf, sps = inp["conf"].numpy(), inp["sps"].numpy()
    a = OS.survival(conf)
    for theta in (0.0, 0.1, 0.5, float(np.median(a)), float(a.max()), 1.0, 2.0, -1.0):
        _check(conf, sps, OS.THRESHOLD, threshold=theta)


def test_schedule_threshold_ragged_with_ties():
    g = np.random.default_rng(14)
    for case in range(20):
        R, gmax = int(g.integers(1, 40)), int(g.integers(1, 17))
        conf = g.choice(np.array([0.25, 0.5, 0.75, 1.0], np.float32), (R, gmax))
        gam = g.integers(0, gmax + 1, R).astype(np.int32)
        sps = g.uniform(0.5, 2.0, R * (gmax + 1)).astype(np.float32)
        for theta in (0.25 ** 3, 0.5, 0.5625, 0.75):   # exactly representable survivals
            _check(conf, sps, OS.THRESHOLD, gam, threshold=theta)


def test_schedule_sts_every_mode():
    """Sequential temperature scaling before the products: calibrated
    survivals and every selection bit-identical to the oracle's."""
    g = np.random.default_rng(15)
    inp = verify_config("headline", device="cpu", V=64)
    conf, sps = inp["conf"].numpy(), inp["sps"].numpy()
    gmax = conf.shape[1]
    temps = g.uniform(0.6, 2.5, gmax).astype(np.float32)
    for mode in MODES:
        _check(conf, sps, mode, sts=temps)
    _check(conf, sps, OS.THRESHOLD, threshold=0.3, sts=temps)
    _check(conf, sps, OS.CAPPED_TOPK, cap=1000, sts=temps)


def test_schedule_sts_limits_and_identity():
    g = np.random.default_rng(16)
    R, gmax = 37, 9
    conf = g.uniform(0.0, 1.0, (R, gmax)).astype(np.float32)
    conf[0, :3] = (0.0, 1.0, 0.5)
    gam = g.integers(0, gmax + 1, R).astype(np.int32)
    sps = g.uniform(0.5, 2.0, R * (gmax + 1)).astype(np.float32)
    for temps in (np.ones(gmax), np.full(gmax, 1e-3), np.full(gmax, 1e3), g.uniform(0.1, 10, gmax)):
        _check(conf, sps, OS.GLOBAL_ARGMAX, gam, sts=temps.astype(np.float32))
    ident = _run(conf, sps, OS.GLOBAL_ARGMAX, gam, sts=np.ones(gmax, np.float32))
    plain = _run(conf, sps, OS.GLOBAL_ARGMAX, gam)
    assert np.array_equal(ident["surv"], plain["surv"])   # T = 1 changes nothing
