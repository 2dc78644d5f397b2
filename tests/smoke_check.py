"""One small pass of the hot path on cuda:0, checked against the oracle."""

import numpy as np
import torch


def run_smoke():
    import draft_verification_amd as sdv
    from oracle import schedule as OS
    from oracle import markov as OM
    from workloads import verify_config, markov_inputs
    from tests.parity_util import oracle_verify_subset, compare_verify, check_stats, to_np, NEAR

    if not torch.cuda.is_available():
        raise RuntimeError("smoke needs a GPU")
    dev = "cuda:0"
    inp = verify_config("tiny", device="cpu")
    inp = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    sched = sdv.sd_schedule(inp["conf"], inp["sps"], sdv.SD_SCHED_EARLY_STOP)
    gpu = sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"],
                        inp["draft_tokens"], sched["ell"], inp["V"], 1.0, inp["seed"],
                        probe=True, stats=True)
    torch.cuda.synchronize()
    ref = OS.schedule(to_np(inp["conf"]), to_np(inp["sps"]), OS.EARLY_STOP)
    assert np.array_equal(to_np(sched["ell"]), ref["ell"]), "schedule mismatch"
    reqs = list(range(inp["R"]))
    ora = oracle_verify_subset(inp, reqs, ref["ell"])
    n_dec, n_near, _ = compare_verify(gpu, ora, reqs)
    check_stats(gpu, ora, reqs, ref["ell"], inp["gmax"])
    # the same verification in rounds that stop at the first rejection, with
    # the draft rows' (m, Z) handed over as a drafter would
    g = inp["gmax"]
    lazy = sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"], inp["draft_tokens"],
                         sched["ell"], inp["V"], 1.0, inp["seed"], stop_at_rejection=True,
                         drf_stats=gpu["row_stats"][:, g + 1:, :].contiguous())
    torch.cuda.synchronize()
    ora_l = oracle_verify_subset(inp, reqs, ref["ell"], stop_at_rejection=True)
    compare_verify(lazy, ora_l, reqs)

    m = markov_inputs(R=3, gamma=3, V=1024, rank=32, H=16, rank_e=8, sigma_f=0.3, device=dev)
    out = sdv.sd_markov_draft(m["U"], m["A"], m["Ct"], m["x0"], m["h"], m["E"], m["w"], 1.0, m["seed"])
    torch.cuda.synchronize()
    f = lambda t: to_np(t).astype(np.float64)
    mref = OM.markov_draft(f(m["U"]), f(m["A"]), f(m["Ct"]).transpose(0, 2, 1), to_np(m["x0"]),
                           f(m["h"]), f(m["E"]), f(m["w"]), 1.0, m["seed"])
    toks = to_np(out["tokens"])
    for r in range(3):
        if not np.array_equal(toks[r], mref["tokens"][r]):
            k = int(np.argmax(toks[r] != mref["tokens"][r]))
            assert mref["dists"][r, k] < NEAR, "markov draft mismatch"
    print(f"smoke ok: {n_dec} verify decisions ({n_near} near-boundary), markov tokens {toks.tolist()}")
