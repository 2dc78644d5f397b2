"""The entry points inside a captured HIP graph: the library enqueues kernels
only (no allocation, copy, memset or synchronisation), so a schedule +
verify step and a drafting call can be captured once and replayed.  Every
replay, with eager work in between, must reproduce the eager outputs bit for
bit (the path is deterministic)."""

import pytest
import torch

import draft_verification_amd as sdv
from workloads import verify_config, markov_inputs

pytestmark = pytest.mark.gpu


def _capture(fn):
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return graph


def _replay_and_compare(graph, outs, ref, n=3):
    for i in range(n):
        for t in outs.values():
            t.fill_(-7 if t.dtype in (torch.int32, torch.int64) else float("nan"))  # eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(outs[k], v), f"replay {i}: {k} differs from the eager call"


def test_schedule_and_verify_step_replays():
    inp = verify_config("mid", device="cuda")
    R, g, V = inp["R"], inp["gmax"], inp["V"]
    dev = "cuda"
    so = dict(ell=torch.empty(R, dtype=torch.int32, device=dev),
              batch=torch.empty(1, dtype=torch.int32, device=dev),
              n_sel=torch.empty(1, dtype=torch.int32, device=dev),
              theta=torch.empty(1, dtype=torch.float64, device=dev),
              surv=torch.empty((R, g), dtype=torch.float32, device=dev))
    vo = dict(n_acc=torch.empty(R, dtype=torch.int32, device=dev),
              tokens=torch.empty((R, g + 1), dtype=torch.int32, device=dev),
              status=torch.empty(R, dtype=torch.int32, device=dev))
    sws = torch.empty(sdv.sd_schedule_workspace_size(R, g), dtype=torch.uint8, device=dev)
    vws = torch.empty(sdv.sd_verify_workspace_size(R, g, V), dtype=torch.uint8, device=dev)

    def step():
        sch = sdv.sd_schedule(inp["conf"], inp["sps"], sdv.SD_SCHED_GLOBAL_ARGMAX, out=so, workspace=sws)
        sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"], inp["draft_tokens"],
                      sch["ell"], V, inp["temperature"], inp["seed"], workspace=vws, out=vo)

    step()
    torch.cuda.synchronize()
    outs = {**{"s_" + k: v for k, v in so.items()}, **{"v_" + k: v for k, v in vo.items()}}
    ref = {k: v.clone() for k, v in outs.items()}
    assert int(ref["v_n_acc"].sum()) >= 0
    graph = _capture(step)
    _replay_and_compare(graph, outs, ref)


def test_verify_in_rounds_replays():
    """Verification that stops at the first rejection (rounds of positions,
    request lists and counters in the workspace, cleared by the kernels
    themselves), with the draft rows' (m, Z) supplied: every replay equals
    the eager call."""
    inp = verify_config("mid", device="cuda")
    R, g, V = inp["R"], inp["gmax"], inp["V"]
    dev = "cuda"
    ell = torch.full((R,), g, dtype=torch.int32, device=dev)
    full = sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"], inp["draft_tokens"], ell,
                         V, inp["temperature"], inp["seed"], stats=True)
    ds = full["row_stats"][:, g + 1:, :].contiguous()
    vo = dict(n_acc=torch.empty(R, dtype=torch.int32, device=dev),
              tokens=torch.empty((R, g + 1), dtype=torch.int32, device=dev),
              status=torch.empty(R, dtype=torch.int32, device=dev))
    vws = torch.empty(sdv.sd_verify_workspace_size(R, g, V), dtype=torch.uint8, device=dev)

    def call():
        sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"], inp["draft_tokens"], ell, V,
                      inp["temperature"], inp["seed"], workspace=vws, out=vo, drf_stats=ds,
                      stop_at_rejection=True)

    call()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in vo.items()}
    graph = _capture(call)
    _replay_and_compare(graph, vo, ref)


def test_markov_draft_replays():
    inp = markov_inputs(R=16, gamma=5, V=4096, rank=64, H=64, rank_e=32, seed=91, device="cuda")
    R, g, V, rank = inp["R"], inp["gamma"], inp["V"], inp["rank"]
    dev = "cuda"
    out = dict(tokens=torch.empty((R, g), dtype=torch.int32, device=dev),
               q_logits=torch.empty((R, g, V), dtype=torch.bfloat16, device=dev),
               conf=torch.empty((R, g), dtype=torch.float32, device=dev),
               status=torch.empty(R, dtype=torch.int32, device=dev))
    ws = torch.empty(max(sdv.sd_markov_draft_workspace_size(R, g, V, rank), 256), dtype=torch.uint8,
                     device=dev)

    def call():
        sdv.sd_markov_draft(inp["U"], inp["A"], inp["Ct"], inp["x0"], inp["h"], inp["E"], inp["w"],
                            inp["temperature"], inp["seed"], workspace=ws, out=out)

    call()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    graph = _capture(call)
    _replay_and_compare(graph, out, ref)
