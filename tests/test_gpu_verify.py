"""GPU parity of sd_verify against the oracle.

Accepted lengths, emitted tokens and status bits must match exactly, except
for requests with a decision the oracle marks near-boundary (distance < 1e-6);
(m, Z) per row and (p(x), q(x)) per tested position within 1e-5 relative.
Where the lengths come from the scheduler, the oracle verifies with the
oracle scheduler's lengths (checked equal to the GPU's); no GPU output is an
oracle input.
"""

import numpy as np
import pytest
import torch

import draft_verification_amd as sdv
from oracle import schedule as OS
from workloads import verify_config, verify_inputs
from tests.parity_util import (oracle_verify_subset, oracle_verify_all, compare_verify, check_stats,
                               check_examined_stats, to_np, VERIFY_TALLY)

pytestmark = pytest.mark.gpu


def _gpu_verify(inp, ell_dev, probe=True, stats=True, alpha=True, **kw):
    out = sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"],
                        inp["draft_tokens"], ell_dev, inp["V"], inp["temperature"], inp["seed"],
                        pos0=inp.get("pos0"), probe=probe, stats=stats, alpha=alpha, **kw)
    torch.cuda.synchronize()
    return out


def _to_cuda(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _full_check(inp, ell, reqs=None, ell_dev=None, ora=None, **kw):
    """ell: host lengths for the oracle (never a GPU output); ell_dev: the
    device lengths the GPU verifies with (default: ell copied over); ora: the
    oracle's result for `reqs` when already computed on the same inputs."""
    ell = np.asarray(ell, np.int64)
    if ell_dev is None:
        ell_dev = torch.as_tensor(ell, dtype=torch.int32, device="cuda")
    gpu = _gpu_verify(inp, ell_dev, **kw)
    R = inp["R"]
    reqs = list(range(R)) if reqs is None else list(reqs)
    ora = oracle_verify_subset(inp, reqs, ell) if ora is None else ora
    n_dec, n_near, mism = compare_verify(gpu, ora, reqs)
    check_stats(gpu, ora, reqs, ell, inp["gmax"])
    _tally(inp, n_dec, n_near, mism)
    return gpu, ora


def _tally(inp, n_dec, n_near, mism):
    """Every divergence is near-boundary (compare_verify asserts it); their
    number is bounded over the whole module by its last test."""
    print(f"decisions={n_dec} near-boundary={n_near} diverged={mism}")
    VERIFY_TALLY.add(inp.get("name", "other shapes"), n_dec, n_near, mism)


@pytest.mark.parametrize("name", ["tiny", "mid"])
@pytest.mark.parametrize("mode", ["full", "early", "argmax"])
def test_verify_workloads(name, mode):
    inp = _to_cuda(verify_config(name, device="cpu"))
    R, g = inp["R"], inp["gmax"]
    if mode == "full":
        _full_check(inp, np.full(R, g))
    else:
        m = OS.EARLY_STOP if mode == "early" else OS.GLOBAL_ARGMAX
        ell_dev = sdv.sd_schedule(inp["conf"], inp["sps"], m)["ell"]
        ref = OS.schedule(to_np(inp["conf"]), to_np(inp["sps"]), m)
        assert np.array_equal(to_np(ell_dev), ref["ell"])
        _full_check(inp, ref["ell"], ell_dev=ell_dev)


def test_verify_ragged_vocab_and_padded_rows():
    # V not a multiple of the 16384-element chunk nor of 64, ld > V, fp32 and bf16
    for dtype in (torch.float32, torch.bfloat16):
        inp = _to_cuda(verify_inputs(R=7, gmax=5, V=40008, ld=40016, dtype=dtype, sigma_t=2.0,
                                     zipf=True, sigma_d=(0.3, 2.0), seed=77))
        _full_check(inp, [0, 1, 2, 3, 4, 5, 5])


def test_verify_vocab_beyond_one_block_per_thread():
    # V > 1024 blocks of 1024: each thread of the correction draw owns a run of
    # two residual blocks; the last chunk and the last block are partial
    for dtype in (torch.bfloat16, torch.float32):
        inp = _to_cuda(verify_inputs(R=4, gmax=2, V=1_050_632, dtype=dtype, sigma_t=2.0,
                                     zipf=True, sigma_d=(1.0, 3.0), seed=82))
        _full_check(inp, [2, 2, 1, 0])


def test_verify_without_drafts():
    """gamma_max = 0: no draft rows, every request samples its one token from
    target row 0 (the bonus draw with l = 0)."""
    for dtype in (torch.bfloat16, torch.float32):
        inp = _to_cuda(verify_inputs(R=6, gmax=0, V=5000, dtype=dtype, sigma_t=2.0, zipf=True, seed=83))
        gpu, _ = _full_check(inp, np.zeros(6))
        assert np.all(to_np(gpu["n_acc"]) == 0)


def test_verify_smallest_vocabulary():
    """V = 8, the smallest the library takes: one 16-byte vector per bf16 row,
    two per fp32 row, a single chunk and block."""
    for dtype in (torch.bfloat16, torch.float32):
        inp = _to_cuda(verify_inputs(R=5, gmax=3, V=8, dtype=dtype, sigma_t=1.5, sigma_d=(0.5, 2.0), seed=84))
        _full_check(inp, np.array([3, 0, 1, 2, 3]))


def test_verify_maximum_draft_length():
    """gamma_max = 255 (the build's limit): 511 batch rows per request and up
    to 255 accept tests at once; drafts close to the target so that long
    prefixes are accepted."""
    inp = _to_cuda(verify_inputs(R=3, gmax=255, V=1024, dtype=torch.bfloat16, sigma_t=2.0,
                                 sigma_d=(0.02, 0.05), seed=84))
    gpu, ora = _full_check(inp, [255, 100, 0])
    assert int(ora["n_acc"].max()) > 20          # the long chains are exercised


def test_verify_vocab_past_the_lds_block_sums():
    """V > 2M: the residual block sums no longer fit in LDS and go through the
    workspace; and V = 2^24, the build's largest vocabulary (1024 chunks)."""
    for R, g, V, dtype, seed in ((2, 2, 4_000_008, torch.bfloat16, 85), (2, 2, 4_000_008, torch.float32, 87),
                                 (1, 1, 1 << 24, torch.bfloat16, 86)):
        inp = _to_cuda(verify_inputs(R=R, gmax=g, V=V, dtype=dtype, sigma_t=2.0, zipf=True,
                                     sigma_d=(1.0, 3.0), seed=seed))
        _full_check(inp, np.full(R, g))


def test_verify_paired_chunks_odd_count_and_ragged_lengths():
    """A bf16 batch large enough for two chunks per bandwidth-pass workgroup
    (R * (2 gamma_max + 1) * chunks >= 16384) with an odd number of chunks
    per row (V = 33576: three chunks, the last pair holding one), and lengths
    from 0 to gamma_max (requests whose whole block is scheduled, and
    requests with slots outside it); sampled requests of every length."""
    R, g, V = 160, 20, 33576
    inp = _to_cuda(verify_inputs(R=R, gmax=g, V=V, dtype=torch.bfloat16, sigma_t=2.0, zipf=True,
                                 sigma_d=(0.5, 2.5), seed=88))
    rng = np.random.default_rng(88)
    ell = rng.integers(0, g + 1, R)
    ell[:8] = g
    reqs = sorted(set([int(i) for i in range(8)] + [int(np.flatnonzero(ell == L)[0]) for L in np.unique(ell)]))
    _, ora = _full_check(inp, ell, reqs=reqs)
    _lazy_check(inp, ell, reqs=reqs, ora=ora)


def test_verify_draws_in_the_request_workgroup():
    """Batches of more than 128 requests make each correction draw inside the
    request's own finishing workgroup (smaller batches of rows of 64 or more
    residual blocks spread the residual sums over the chip): fp32 rows in one
    pass and in rounds, and bf16 rows past the LDS block sums (V > 2M) on
    sampled requests."""
    inp = _to_cuda(verify_inputs(R=130, gmax=3, V=5000, dtype=torch.float32, sigma_t=2.0,
                                 sigma_d=(0.5, 3.0), seed=91))
    _full_check(inp, np.full(130, 3))
    _lazy_check(inp, np.full(130, 3))
    inp = verify_inputs(R=130, gmax=1, V=2_100_000, dtype=torch.bfloat16, sigma_t=2.0, zipf=True,
                        sigma_d=(1.0, 3.0), seed=92, device="cuda")
    gpu, _ = _full_check(inp, np.full(130, 1), reqs=[0, 1, 64, 129])
    assert np.all(to_np(gpu["status"]) == 0)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 151936), (torch.float32, 70000)])
def test_verify_draws_identical_in_either_path(dtype, V):
    """The first 128 requests of a 129-request batch verified alone (draws
    spread over the chip: rows of 149 and 69 residual blocks) and inside the
    batch (each draw in its request's workgroup): identical outputs, bit for
    bit, in one pass and in rounds."""
    R, g = 129, 6
    inp = verify_inputs(R=R, gmax=g, V=V, dtype=dtype, sigma_t=3.0, zipf=True, sigma_d=(0.5, 3.0),
                        seed=93, device="cuda")
    ell = torch.full((R,), g, dtype=torch.int32, device="cuda")
    for lazy in (False, True):
        outs = []
        for n in (R, R - 1):
            o = sdv.sd_verify(inp["tgt"], inp["tgt_row0"][:n], inp["drf"], inp["drf_row0"][:n],
                              inp["draft_tokens"][:n].contiguous(), ell[:n], V, 1.0, inp["seed"],
                              probe=True, stats=True, stop_at_rejection=lazy)
            torch.cuda.synchronize()
            outs.append({k: to_np(v)[:R - 1] for k, v in o.items() if v is not None})
        for k in outs[0]:
            assert np.array_equal(outs[0][k], outs[1][k], equal_nan=True), (lazy, k)
        assert np.all(outs[0]["status"] == 0)


def test_verify_temperature_and_positions():
    inp = _to_cuda(verify_inputs(R=9, gmax=6, V=20000, dtype=torch.bfloat16, sigma_t=2.5,
                                 zipf=True, sigma_d=(0.5, 2.5), seed=78, temperature=0.7))
    inp["pos0"] = torch.arange(9, dtype=torch.int64, device="cuda") * 1000 + 17
    _full_check(inp, np.full(9, 6))


@pytest.mark.parametrize("T", [0.05, 4.0])
def test_verify_low_and_high_temperature(T):
    """T = 0.05 (rows nearly one-hot: logits / T span hundreds of units, the
    exponentials of everything but the top few underflow) and T = 4 (rows
    nearly flat); drafts drawn at the same temperature; in one pass and in
    rounds."""
    for dtype in (torch.bfloat16, torch.float32):
        inp = _to_cuda(verify_inputs(R=8, gmax=5, V=30000, dtype=dtype, sigma_t=2.5, zipf=True,
                                     sigma_d=(0.2, 2.0), seed=91, temperature=T))
        ell = np.array([5, 5, 4, 5, 3, 5, 5, 1])
        full, _ = _full_check(inp, ell)
        lazy, _ = _lazy_check(inp, ell)
        for k in ("n_acc", "tokens", "status"):
            assert torch.equal(lazy[k], full[k]), k


def test_verify_packed_layout():
    # rows of consecutive requests packed back to back (no reserved slots)
    inp = _to_cuda(verify_inputs(R=6, gmax=4, V=4096, dtype=torch.bfloat16, sigma_t=2.0,
                                 seed=79))
    ell_h = np.array([4, 0, 2, 3, 1, 4])
    t0 = np.concatenate([[0], np.cumsum(ell_h + 1)[:-1]])
    d0 = np.concatenate([[0], np.cumsum(ell_h)[:-1]])
    tgt = torch.cat([inp["tgt"][r * 5:r * 5 + ell_h[r] + 1] for r in range(6)])
    drf = torch.cat([inp["drf"][r * 4:r * 4 + ell_h[r]] for r in range(6)])
    inp.update(tgt=tgt.contiguous(), drf=drf.contiguous(),
               tgt_row0=torch.as_tensor(t0, dtype=torch.int32, device="cuda"),
               drf_row0=torch.as_tensor(d0, dtype=torch.int32, device="cuda"))
    _full_check(inp, ell_h)


@pytest.fixture(scope="module")
def headline():
    """R=256, gamma=11, V=151936 bf16 at the full block, as timed by bench.py:
    the inputs, the GPU's and the oracle's schedules (global argmax), and the
    oracle's verification of every request on the oracle's lengths."""
    inp = verify_config("headline", device="cuda")
    R, g = inp["R"], inp["gmax"]
    sched = sdv.sd_schedule(inp["conf"], inp["sps"], OS.GLOBAL_ARGMAX)
    ref = OS.schedule(to_np(inp["conf"]), to_np(inp["sps"]), OS.GLOBAL_ARGMAX)
    assert np.array_equal(to_np(sched["ell"]), ref["ell"])
    assert ref["B"] == R * (g + 1)   # the global argmax takes the full block
    ora = oracle_verify_all(inp, ref["ell"])
    return inp, ref["ell"], sched["ell"], ora


def test_verify_headline_full_block(headline):
    """Every request of the headline block against the oracle: lengths,
    tokens, statuses, (m, Z) of all 5888 rows, p(x), q(x) and alpha."""
    inp, ell, ell_dev, ora = headline
    gpu, _ = _full_check(inp, ell, ell_dev=ell_dev, ora=ora)
    assert np.all(to_np(gpu["status"]) == 0)


@pytest.fixture(scope="module")
def ragged():
    """R=512, gamma_r in 1..16, reserved slots past gamma_r hold NaN; the
    async capacity chain (global argmax on the previous confidences, then the
    top K of the current ones) on the GPU and in the oracle, and the oracle's
    verification of every request on the oracle's lengths."""
    inp = verify_config("ragged", device="cuda")
    first = sdv.sd_schedule(inp["conf_prev"], inp["sps"], OS.GLOBAL_ARGMAX, gamma_r=inp["gamma_r"])
    sched = sdv.sd_schedule(inp["conf"], inp["sps"], OS.CAPPED_TOPK, gamma_r=inp["gamma_r"],
                            cap_k=first["n_sel"])
    ref = OS.async_schedule(to_np(inp["conf"]), to_np(inp["conf_prev"]), to_np(inp["sps"]),
                            to_np(inp["gamma_r"]))
    assert np.array_equal(to_np(sched["ell"]), ref["ell"])
    ora = oracle_verify_all(inp, ref["ell"])
    return inp, ref["ell"], sched["ell"], ora


def test_verify_ragged_async(ragged):
    """Every one of the 512 requests against the oracle, in one pass and in
    rounds stopping at each request's first rejection."""
    inp, ell, ell_dev, ora = ragged
    gpu, _ = _full_check(inp, ell, ell_dev=ell_dev, ora=ora)
    assert np.all(to_np(gpu["status"]) == 0)   # no NaN slot was read
    assert len(set(to_np(inp["gamma_r"]).tolist())) == inp["gmax"]   # every draft length occurs
    lazy, _ = _lazy_check(inp, ell, ell_dev=ell_dev, ora=ora)
    for k in ("n_acc", "tokens", "status"):
        assert torch.equal(lazy[k], gpu[k]), k


def test_verify_degenerate_rows_and_tokens():
    V, g = 2048, 3
    inp = _to_cuda(verify_inputs(R=8, gmax=g, V=V, dtype=torch.float32, sigma_t=2.0, seed=80))
    tgt, drf, toks = inp["tgt"], inp["drf"], inp["draft_tokens"]
    tgt[0 * 4 + 1, 10] = float("nan")                # r0: NaN in a needed target row
    tgt[1 * 4 + 3, :] = float("-inf")               # r1: bonus row all -inf
    toks[2, 0] = V + 5                              # r2: bad token at position 1
    drf[3 * 3 + 0, int(toks[3, 0])] = float("-inf")  # r3: q(x) = 0 at position 1
    tgt[4 * 4 + 2, 0] = float("inf")                # r4: +inf in a needed row
    tgt[5 * 4 + 3, 0] = float("nan")                # r5: NaN only past l_r -> unread
    drf[6 * 3:6 * 3 + 3] = tgt[6 * 4:6 * 4 + 3]     # r6: p == q everywhere
    gpu, ora = _full_check(inp, [3, 3, 3, 3, 3, 2, 3, 0])
    st = to_np(gpu["status"])
    assert st[0] == sdv.SD_ST_NONFINITE and st[1] == sdv.SD_ST_ZERO_Z
    assert st[2] & sdv.SD_ST_BAD_TOKEN and st[3] & sdv.SD_ST_ZERO_Q
    assert st[4] == sdv.SD_ST_NONFINITE and st[5] == 0
    assert to_np(gpu["n_acc"])[6] == 3


def test_verify_repeatable():
    inp = _to_cuda(verify_config("mid", device="cpu"))
    ell = torch.full((inp["R"],), inp["gmax"], dtype=torch.int32, device="cuda")
    a = _gpu_verify(inp, ell)
    b = _gpu_verify(inp, ell)
    for k in ("n_acc", "tokens", "status", "probe", "row_stats", "alpha"):
        assert torch.equal(a[k], b[k]), k


def test_verify_host_errors():
    inp = _to_cuda(verify_inputs(R=2, gmax=2, V=64, dtype=torch.float32, seed=81))
    ell = torch.full((2,), 2, dtype=torch.int32, device="cuda")
    with pytest.raises(sdv.SdvError):
        sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"],
                      inp["draft_tokens"], ell, 60, 1.0, 1)           # V % 8 != 0
    with pytest.raises(sdv.SdvError):
        sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"],
                      inp["draft_tokens"], ell, 64, 0.0, 1)           # temperature 0
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_verify(inp["tgt"], inp["tgt_row0"], inp["drf"], inp["drf_row0"],
                      inp["draft_tokens"], ell, 64, 1.0, 1, workspace=small)
    assert e.value.code == -2


def _draft_stats(gpu, gmax):
    """The draft rows' (m, Z) as a call that read them reported them (row_stats
    slots gmax+1..2*gmax): the pairs a drafter hands over."""
    return gpu["row_stats"][:, gmax + 1:, :].contiguous()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_verify_with_draft_statistics(dtype):
    """The drafter's (m, Z) in place of the pass over the draft rows: the
    oracle (which reads the rows) still agrees, the target rows' statistics
    are those of the full pass, and the supplied pairs are what row_stats
    reports for the draft slots.  T = 0.8 and positions offset."""
    inp = _to_cuda(verify_inputs(R=9, gmax=6, V=40008, ld=40016, dtype=dtype, sigma_t=2.0,
                                 zipf=True, sigma_d=(0.3, 2.5), seed=88, temperature=0.8))
    inp["pos0"] = torch.arange(9, dtype=torch.int64, device="cuda") * 13
    g = inp["gmax"]
    ell = np.array([6, 5, 0, 1, 6, 3, 6, 2, 4])
    full, _ = _full_check(inp, ell)
    ds = _draft_stats(full, g)
    gpu, _ = _full_check(inp, ell, drf_stats=ds)
    rs_full, rs, ds_h = to_np(full["row_stats"]), to_np(gpu["row_stats"]), to_np(ds)
    for r, L in enumerate(ell):
        assert np.array_equal(rs[r, :L + 1], rs_full[r, :L + 1])
        assert np.array_equal(rs[r, g + 1:g + 1 + L], ds_h[r, :L])


def test_verify_degenerate_draft_statistics():
    """Pairs that encode an all -inf row or a row holding NaN fail the request
    exactly as reading the row does; pairs outside the documented domain
    (Z = 0, Z = inf, m = +inf) fail it as NONFINITE."""
    V, g, R = 2048, 3, 6
    inp = _to_cuda(verify_inputs(R=R, gmax=g, V=V, dtype=torch.float32, sigma_t=2.0, seed=89))
    inp["drf"][0 * g + 1, :] = float("-inf")   # r0: draft row 2 all -inf
    inp["drf"][1 * g + 0, 7] = float("nan")    # r1: NaN in draft row 1
    ell = np.full(R, g)
    full, _ = _full_check(inp, ell)
    st_full = to_np(full["status"])
    assert st_full[0] == sdv.SD_ST_ZERO_Z and st_full[1] == sdv.SD_ST_NONFINITE
    ds = _draft_stats(full, g).clone()
    ds[2, 0] = torch.tensor([1.0, 0.0])
    ds[3, 1] = torch.tensor([1.0, float("inf")])
    ds[4, 2] = torch.tensor([float("inf"), 1.0])
    gpu, _ = _full_check(inp, ell, reqs=[0, 1, 5], drf_stats=ds)
    st, n_acc, toks = to_np(gpu["status"]), to_np(gpu["n_acc"]), to_np(gpu["tokens"])
    for r in (2, 3, 4):
        assert st[r] == sdv.SD_ST_NONFINITE and n_acc[r] == 0 and np.all(toks[r] == -1)


def test_verify_headline_with_draft_statistics(headline):
    """The headline block with the draft rows' statistics supplied (only the
    3072 target rows are streamed): every request against the oracle."""
    inp, ell, ell_dev, ora = headline
    g = inp["gmax"]
    full = _gpu_verify(inp, ell_dev, probe=False, alpha=False)
    gpu, _ = _full_check(inp, ell, ell_dev=ell_dev, ora=ora, drf_stats=_draft_stats(full, g))
    assert np.all(to_np(gpu["status"]) == 0)


def _lazy_check(inp, ell, reqs=None, ell_dev=None, ora=None, **kw):
    """Verification that stops at each request's first rejection against the
    oracle that reads positions in order; statistics of the rows the oracle
    examined.  ora: an oracle result for `reqs` already computed on the same
    inputs and lengths (the one-pass oracle gives the same lengths, tokens,
    statuses and decisions on usable rows, and the statistics of every row,
    of which the examined ones are compared)."""
    ell = np.asarray(ell, np.int64)
    if ell_dev is None:
        ell_dev = torch.as_tensor(ell, dtype=torch.int32, device="cuda")
    gpu = _gpu_verify(inp, ell_dev, alpha=False, stop_at_rejection=True, **kw)
    reqs = list(range(inp["R"])) if reqs is None else list(reqs)
    if ora is None:
        ora = oracle_verify_subset(inp, reqs, ell, stop_at_rejection=True)
    n_dec, n_near, mism = compare_verify(gpu, ora, reqs)
    check_examined_stats(gpu, ora, reqs, ell, inp["gmax"])
    _tally(inp, n_dec, n_near, mism)
    return gpu, ora


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_verify_stop_at_rejection_workloads(name):
    """Same lengths and tokens as reading every row (usable rows), and the
    oracle's in-order procedure agrees; full block and early-stop lengths."""
    inp = _to_cuda(verify_config(name, device="cpu"))
    R, g = inp["R"], inp["gmax"]
    ref = OS.schedule(to_np(inp["conf"]), to_np(inp["sps"]), OS.EARLY_STOP)
    for ell in (np.full(R, g), ref["ell"]):
        gpu, _ = _lazy_check(inp, ell)
        full = _gpu_verify(inp, torch.as_tensor(ell, dtype=torch.int32, device="cuda"), alpha=False)
        for k in ("n_acc", "tokens", "status"):
            assert torch.equal(gpu[k], full[k]), k


def test_verify_stop_at_rejection_ragged_and_long_chains():
    """Ragged vocabulary, padded rows, fp32 and bf16; gamma_max = 255 with
    drafts close to the targets, so that the eight rounds of positions
    (2, 6, 14, ..., 256) are all used; gamma_max = 0."""
    for dtype in (torch.float32, torch.bfloat16):
        inp = _to_cuda(verify_inputs(R=7, gmax=5, V=40008, ld=40016, dtype=dtype, sigma_t=2.0,
                                     zipf=True, sigma_d=(0.3, 2.0), seed=77))
        _lazy_check(inp, [0, 1, 2, 3, 4, 5, 5])
    inp = _to_cuda(verify_inputs(R=3, gmax=255, V=1024, dtype=torch.bfloat16, sigma_t=2.0,
                                 sigma_d=(0.02, 0.05), seed=84))
    _, ora = _lazy_check(inp, [255, 100, 0])
    assert int(ora["n_acc"].max()) > 30
    inp = _to_cuda(verify_inputs(R=6, gmax=0, V=5000, dtype=torch.bfloat16, sigma_t=2.0, zipf=True, seed=83))
    _lazy_check(inp, np.zeros(6))


def test_verify_stop_at_rejection_vocab_past_the_lds_block_sums():
    inp = _to_cuda(verify_inputs(R=2, gmax=2, V=4_000_008, dtype=torch.bfloat16, sigma_t=2.0, zipf=True,
                                 sigma_d=(1.0, 3.0), seed=85))
    _lazy_check(inp, [2, 2])


def test_verify_stop_at_rejection_ignores_rows_past_the_rejection():
    """Rows past each request's first rejection spoiled with NaN / -inf: the
    result is that of the clean rows (reading every row fails those
    requests); an unusable row at the rejected position, or an unusable bonus
    row after full acceptance, fails the request."""
    V, g, R = 4096, 6, 12
    inp = _to_cuda(verify_inputs(R=R, gmax=g, V=V, dtype=torch.float32, sigma_t=2.0, sigma_d=(0.5, 2.5),
                                 seed=90))
    ell = np.array([6, 6, 6, 5, 6, 4, 6, 6, 3, 6, 6, 2])
    clean, _ = _lazy_check(inp, ell)
    n_acc = to_np(clean["n_acc"])
    tgt, drf = inp["tgt"], inp["drf"]
    spoiled = []
    for r in range(R):
        n, L = int(n_acc[r]), int(ell[r])
        if n < L - 1:                                  # rows past position n + 1 exist
            tgt[r * (g + 1) + n + 1:r * (g + 1) + L + 1] = float("nan")
            drf[r * g + n + 1:r * g + L] = float("-inf")
            spoiled.append(r)
    assert len(spoiled) >= 3
    gpu, _ = _lazy_check(inp, ell)
    for k in ("n_acc", "tokens", "status"):
        assert torch.equal(gpu[k], clean[k]), k
    full = _gpu_verify(inp, torch.as_tensor(ell, dtype=torch.int32, device="cuda"), alpha=False)
    assert all(to_np(full["status"])[r] & sdv.SD_ST_NONFINITE for r in spoiled)
    # an unusable row at the rejected position, and an unusable bonus row
    r = spoiled[0]
    inp["tgt"][r * (g + 1) + int(n_acc[r]), 0] = float("nan")
    acc = [q for q in range(R) if n_acc[q] == ell[q]]
    if acc:
        inp["tgt"][acc[0] * (g + 1) + int(ell[acc[0]])] = float("-inf")
    gpu, _ = _lazy_check(inp, ell)
    st = to_np(gpu["status"])
    assert st[r] == sdv.SD_ST_NONFINITE
    if acc:
        assert st[acc[0]] == sdv.SD_ST_ZERO_Z


def test_verify_headline_stop_at_rejection(headline):
    """The headline block read in rounds, with and without the drafter's
    statistics: every request against the oracle."""
    inp, ell, ell_dev, ora = headline
    g = inp["gmax"]
    full = _gpu_verify(inp, ell_dev, probe=False, alpha=False)
    gpu, _ = _lazy_check(inp, ell, ell_dev=ell_dev, ora=ora)
    for k in ("n_acc", "tokens", "status"):
        assert torch.equal(gpu[k], full[k]), k
    gpu2, _ = _lazy_check(inp, ell, ell_dev=ell_dev, ora=ora, drf_stats=_draft_stats(full, g))
    for k in ("n_acc", "tokens", "status"):
        assert torch.equal(gpu2[k], full[k]), k


def test_verify_zz_decision_tally():
    """Over every verify decision the tests of this module compared (the
    named workloads at full size on every request, and the special shapes):
    each divergence was near-boundary, and divergences stay within 0.01 % of
    the decisions.  The near-boundary share is reported per workload."""
    if not VERIFY_TALLY.rows:
        pytest.skip("no verify decisions were compared in this session")
    n_dec, n_near, n_div = VERIFY_TALLY.check()
    by = {}
    for what, d, nr, dv in VERIFY_TALLY.rows:
        t = by.setdefault(what, [0, 0, 0])
        t[0] += d
        t[1] += nr
        t[2] += dv
    for what, (d, nr, dv) in sorted(by.items()):
        print(f"{what}: decisions={d} near-boundary={nr} ({nr / max(d, 1):.3%}) diverged={dv}")
    print(f"all: decisions={n_dec} near-boundary={n_near} ({n_near / max(n_dec, 1):.3%}) diverged={n_div}")
