"""Every entry point on a stream other than torch's current one.

The binding allocates outputs and the temporary workspace on the stream the
kernels run on, so that a block freed on return is never handed to another
stream's work while those kernels may still use it.  Each call on a side
stream, with the default stream kept busy allocating and filling memory in the
meantime, must give the outputs of the same call on the default stream."""

import pytest
import torch

import draft_verification_amd as sdv
from workloads import verify_config, markov_inputs, rnn_inputs

pytestmark = pytest.mark.gpu


def _churn():
    """Allocate, fill and free memory on the default stream."""
    for i in range(8):
        t = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
        t.fill_(i)
        del t


def _same(a, b):
    for k, v in a.items():
        if v is None:
            assert b[k] is None, k
        else:
            assert torch.equal(v, b[k]), k


def _on_side(fn):
    """fn(side) with the side stream ordered after everything enqueued so far
    on the default stream (inputs included), then the default stream churns
    memory while the side stream runs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = fn(side)
    _churn()
    side.synchronize()
    torch.cuda.current_stream().wait_stream(side)
    return out


def test_schedule_and_verify_on_a_side_stream():
    inp = verify_config("mid", device="cuda")
    R, g, V = inp["R"], inp["gmax"], inp["V"]

    def run(stream):
        sch = sdv.sd_schedule(inp["conf"], inp["sps"], sdv.SD_SCHED_GLOBAL_ARGMAX, stream=stream)
        ver = sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"], inp["draft_tokens"],
                            sch["ell"], V, inp["temperature"], inp["seed"], probe=True, stats=True,
                            alpha=True, stream=stream)
        lazy = sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"],
                             inp["draft_tokens"], sch["ell"], V, inp["temperature"], inp["seed"],
                             stop_at_rejection=True, stream=stream)
        return sch, ver, lazy

    ref = run(None)
    torch.cuda.synchronize()
    got = _on_side(run)
    for a, b in zip(ref, got):
        _same(a, b)
    req = torch.arange(R, dtype=torch.int64, device="cuda")
    pos = req + 1
    u_ref = sdv.sd_uniforms(inp["seed"], req, pos, 1)
    u_side = _on_side(lambda s: sdv.sd_uniforms(inp["seed"], req, pos, 1, stream=s))
    assert torch.equal(u_ref, u_side)


def test_drafting_heads_on_a_side_stream():
    mk = markov_inputs(R=20, gamma=4, V=4096, rank=64, H=64, rank_e=32, sigma_f=0.3, seed=101,
                       device="cuda")
    run = lambda s: sdv.sd_markov_draft(mk["U"], mk["A"], mk["Ct"], mk["x0"], mk["h"], mk["E"], mk["w"],
                                        1.0, mk["seed"], stats=True, stream=s)
    ref = run(None)
    torch.cuda.synchronize()
    _same(ref, _on_side(run))
    rn = rnn_inputs(R=20, gamma=4, V=4096, d=64, H=64, rank_e=32, seed=102, device="cuda")
    run = lambda s: sdv.sd_rnn_draft(rn["U"], rn["W"], rn["Es"], rn["Ct"], rn["x0"], rn["h"], rn["E"],
                                     rn["w"], 1.0, rn["seed"], stats=True, stream=s)
    ref = run(None)
    torch.cuda.synchronize()
    _same(ref, _on_side(run))


def test_budget_planner_on_a_side_stream():
    R, G = 32, 6
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    alpha = torch.rand((R, G), generator=g, device="cuda")
    ell = torch.randint(0, G + 1, (R,), generator=g, device="cuda", dtype=torch.int32)
    status = torch.zeros(R, dtype=torch.int32, device="cuda")
    sps = torch.linspace(1.0, 50.0, R * (G + 1), device="cuda")
    cost = torch.full((G,), 1e-3, device="cuda")

    def state():   # made on the default stream before the side stream waits for it
        return (torch.full((G,), 0.5, dtype=torch.float64, device="cuda"),
                torch.zeros(G, dtype=torch.int64, device="cuda"))

    def run(stream, ema, cnt):
        sdv.sd_lightspec_update(alpha, ell, status, 0.2, ema, cnt, stream=stream)
        plan = sdv.sd_lightspec_plan(ema, cnt, ell, sps, cost, stream=stream)
        return dict(plan, ema=ema, cnt=cnt)

    ref = run(None, *state())
    torch.cuda.synchronize()
    ema, cnt = state()
    _same(ref, _on_side(lambda s: run(s, ema, cnt)))
