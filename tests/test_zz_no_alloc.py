"""sd_verify_noalloc, the entry point that allocates nothing, against
sd_verify: two calls in a row on one GPU (the headline block, then the tiny
workload, smaller), in one pass and in rounds; every output bit for bit
equal to sd_verify's on the same inputs.  Sizes past the library's
workspace are refused on the host."""

import pytest
import torch

import draft_verification_amd as sdv
from workloads import verify_config

pytestmark = pytest.mark.gpu


def _outs(R, g, dev="cuda"):
    return dict(n_acc=torch.full((R,), -9, dtype=torch.int32, device=dev),
                tokens=torch.full((R, g + 1), -9, dtype=torch.int32, device=dev),
                status=torch.full((R,), -9, dtype=torch.int32, device=dev),
                probe=torch.full((R, g, 2), -9.0, device=dev),
                row_stats=torch.full((R, 2 * g + 1, 2), -9.0, device=dev),
                alpha=torch.full((R, g), -9.0, device=dev))


def _both(inp, lazy):
    R, g, V = inp["R"], inp["gmax"], inp["V"]
    ell = torch.full((R,), g, dtype=torch.int32, device="cuda")
    ref_o, got_o = _outs(R, g), _outs(R, g)
    if lazy:   # acceptance rates need every row: not with the rounds
        ref_o.pop("alpha")
        got_o.pop("alpha")
    sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"], inp["draft_tokens"], ell, V,
                  inp["temperature"], inp["seed"], stop_at_rejection=lazy, out=ref_o, probe=True,
                  stats=True, alpha=not lazy)
    sdv.sd_verify_noalloc(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"], inp["draft_tokens"],
                          ell, V, inp["temperature"], inp["seed"], stop_at_rejection=lazy, out=got_o)
    torch.cuda.synchronize()
    for k in ref_o:
        assert torch.equal(ref_o[k], got_o[k]), (inp["name"], lazy, k)
    assert torch.all(got_o["status"] == 0)


def test_noalloc_equals_sd_verify_on_two_calls_in_a_row():
    """The headline block (R=256, gamma=11, V=151936 bf16), then the tiny
    workload (R=4, gamma=4, V=1024 fp32): the second call runs on the
    workspace the first one left behind."""
    big = verify_config("headline", device="cuda")
    small = verify_config("tiny", device="cuda")
    assert (sdv.sd_verify_workspace_size(small["R"], small["gmax"], small["V"])
            < sdv.sd_verify_workspace_size(big["R"], big["gmax"], big["V"]))
    for lazy in (False, True):
        _both(big, lazy)
        _both(small, lazy)
