"""Synthetic workloads for scheduling, verification and Markov drafting.

Recipes (random draws only; torch generators seeded per workload, on whatever
device the caller names - the same seed gives different numbers on CPU and GPU,
so a parity test always hands the *same tensors* to both sides):

* target logit rows t: N(0, sigma_t^2), optionally plus a Zipf(1.1) rank
  offset -1.1 * ln(rank), rank 1 being the row's own largest draw (this gives
  the heavy-tailed rows with top-1 mass of roughly 0.3-0.9 the headline
  workload describes);
* draft rows d = t + N(0, sigma_d^2), sigma_d per request when a range is
  given; the draft row of position j perturbs the target row of position j;
* both rounded to the logit dtype (bf16 or fp32);
* draft tokens drawn from the draft rows by the Gumbel-max trick
  (argmax of d / T + Gumbel noise) with torch's generator - an input recipe,
  independent of the counter hash the method itself uses;
* confidences sigmoid(N(mu_k, 1)), throughput tables
  SPS(B) = B / (1 + B / B_sat) * (1 + A * saw_P(B)), saw_P(B) = ((B-1) mod P) / (P/2) - 1;
* the reserved-slot layout: request r owns target rows r*(g+1) .. and draft
  rows r*g ..; slots past a request's drafted length are filled with NaN so
  that any read of them shows up as a non-finite row.
"""

import math

import torch

# Workload table (sizes as the workloads are described; V multiples of 8).
CONFIGS = {
    "tiny": dict(R=4, gmax=4, V=1024, dtype=torch.float32, sigma_t=2.0, zipf=False,
                 sigma_d=(1.0, 1.0), conf_mu=lambda k: 1.0, sps=(32, 0.05, 8), seed_off=1),
    "mid": dict(R=64, gmax=8, V=32000, dtype=torch.bfloat16, sigma_t=2.5, zipf=True,
                sigma_d=(1.5, 1.5), conf_mu=lambda k: 1.5, sps=(256, 0.08, 64), seed_off=2),
    "headline": dict(R=256, gmax=11, V=151936, dtype=torch.bfloat16, sigma_t=3.0, zipf=True,
                     sigma_d=(0.5, 3.0), conf_mu=lambda k: 2.0 - 0.2 * k, sps=(256, 0.08, 64),
                     seed_off=3),
    "ragged": dict(R=512, gmax=16, V=151936, dtype=torch.bfloat16, sigma_t=3.0, zipf=True,
                   sigma_d=(0.5, 3.0), conf_mu=lambda k: 2.0 - 0.2 * k, sps=(256, 0.08, 64),
                   seed_off=5, ragged=True),
}
MARKOV = dict(R=128, gamma=16, V=129280, rank=256, H=4096, rank_e=256, sigma_u=2.0,
              sigma_f=0.02, sps=(256, 0.08, 64), seed_off=4)

RNN = dict(R=128, gamma=16, V=129280, d=128, H=4096, rank_e=256, sigma_u=2.0, sigma_w=0.5,
           sigma_e=1.0, sigma_c=0.05, sigma_f=0.02, seed_off=5)

BASE_SEED = 20261202
SAMPLE_SEED = 0xC0FFEE


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def sps_table(n, b_sat, amp, period):
    """fp32 table, entry B-1 for batch B = 1..n."""
    B = torch.arange(1, n + 1, dtype=torch.float64)
    saw = torch.remainder(B - 1, period) / (period / 2.0) - 1.0
    return (B / (1.0 + B / b_sat) * (1.0 + amp * saw)).to(torch.float32)


def _zipf_rows(x, s=1.1, chunk=256):
    """x - s * ln(rank) with rank 1 = the row's largest entry (in place, chunked)."""
    V = x.shape[1]
    logr = torch.log(torch.arange(1, V + 1, device=x.device, dtype=torch.float32)) * s
    for i in range(0, x.shape[0], chunk):
        blk = x[i:i + chunk]
        order = torch.argsort(blk, dim=1, descending=True)
        off = torch.empty_like(blk)
        off.scatter_(1, order, logr.expand(blk.shape[0], V).contiguous())
        blk -= off
    return x


def _normal(shape, std, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _gumbel_argmax(d, T, g, chunk=1024):
    """One token per row drawn from softmax(d / T) by Gumbel-max."""
    out = torch.empty(d.shape[0], dtype=torch.int32, device=d.device)
    for i in range(0, d.shape[0], chunk):
        blk = d[i:i + chunk].float() / T
        u = torch.rand(blk.shape, generator=g, device=d.device, dtype=torch.float32)
        u.clamp_(min=1e-30, max=1.0 - 1e-7)
        out[i:i + chunk] = torch.argmax(blk - torch.log(-torch.log(u)), dim=1).to(torch.int32)
    return out


def verify_inputs(R, gmax, V, dtype=torch.bfloat16, sigma_t=2.0, zipf=False,
                  sigma_d=(1.0, 1.0), conf_mu=lambda k: 1.0, sps=(32, 0.05, 8),
                  gamma_r=None, seed=BASE_SEED, device="cpu", temperature=1.0,
                  ld=None, with_prev=False):
    """Inputs for one schedule + verify step in the reserved-slot layout.

    Returns a dict of tensors on ``device``: tgt [R*(gmax+1)][ld], drf
    [max(R*gmax,1)][ld], tgt_row0, drf_row0 [R] int32, draft_tokens [R][gmax]
    int32, conf (and conf_prev) [R][gmax] fp32, gamma_r [R] int32, sps fp32,
    plus the scalars R, gmax, V, ld, temperature, seed (sampling), pos0.
    """
    g = _gen(device, seed)
    ld = V if ld is None else ld
    if gamma_r is None:
        gam = torch.full((R,), gmax, dtype=torch.int32)
    else:
        gam = torch.as_tensor(gamma_r, dtype=torch.int32)
    nt, nd = R * (gmax + 1), max(R * gmax, 1)
    tgt = torch.empty((nt, ld), dtype=dtype, device=device)
    drf = torch.empty((nd, ld), dtype=dtype, device=device)
    if ld > V:
        tgt[:, V:] = 0
        drf[:, V:] = 0
    lo, hi = sigma_d
    sig = lo + (hi - lo) * torch.rand((R,), generator=g, device=device, dtype=torch.float32)
    chunk_req = max(1, 4096 // (gmax + 1))
    for r0 in range(0, R, chunk_req):
        r1 = min(R, r0 + chunk_req)
        n = (r1 - r0) * (gmax + 1)
        t = _normal((n, V), sigma_t, g, device)
        if zipf:
            _zipf_rows(t)
        t3 = t.view(r1 - r0, gmax + 1, V)
        tgt[r0 * (gmax + 1):r1 * (gmax + 1), :V] = t.to(dtype)
        if gmax > 0:
            d = t3[:, :gmax, :] + _normal((r1 - r0, gmax, V), 1.0, g, device) * sig[r0:r1, None, None]
            drf[r0 * gmax:r1 * gmax, :V] = d.reshape(-1, V).to(dtype)
        del t, t3
    # draft tokens from the (rounded) draft rows
    if gmax > 0:
        toks = _gumbel_argmax(drf[:R * gmax, :V], temperature, g).view(R, gmax)
    else:
        toks = torch.zeros((R, 0), dtype=torch.int32, device=device)
    mus = torch.tensor([conf_mu(k) for k in range(1, gmax + 1)], dtype=torch.float32)
    conf = torch.sigmoid(_normal((R, gmax), 1.0, g, device) + mus.to(device))
    conf_prev = torch.sigmoid(_normal((R, gmax), 1.0, g, device) + mus.to(device)) if with_prev else None
    # reserved slots past gamma_r hold NaN: never read
    gam_d = gam.to(device)
    if gamma_r is not None and gmax > 0:
        for r in torch.nonzero(gam < gmax).flatten().tolist():
            gr = int(gam[r])
            tgt[r * (gmax + 1) + gr + 1:(r + 1) * (gmax + 1), :V] = float("nan")
            drf[r * gmax + gr:(r + 1) * gmax, :V] = float("nan")
            toks[r, gr:] = -7
    b_sat, amp, period = sps
    table = sps_table(R * (gmax + 1), b_sat, amp, period).to(device)
    return dict(
        R=R, gmax=gmax, V=V, ld=ld, temperature=temperature, seed=SAMPLE_SEED, pos0=None,
        tgt=tgt, drf=drf,
        tgt_row0=(torch.arange(R, dtype=torch.int32) * (gmax + 1)).to(device),
        drf_row0=(torch.arange(R, dtype=torch.int32) * gmax).to(device),
        draft_tokens=toks.contiguous(), conf=conf.contiguous(), conf_prev=conf_prev,
        gamma_r=gam_d, sps=table,
    )


def verify_config(name, device="cpu", data_shift=0, **over):
    """One of the named schedule + verify workloads; data_shift != 0 draws an
    independent input set of the same workload."""
    cfg = dict(CONFIGS[name])
    ragged = cfg.pop("ragged", False)
    seed_off = cfg.pop("seed_off")
    cfg.update(over)
    seed = BASE_SEED + seed_off + 1000003 * data_shift
    if ragged and "gamma_r" not in over:
        g = _gen("cpu", seed + 1000)
        cfg["gamma_r"] = torch.randint(1, cfg["gmax"] + 1, (cfg["R"],), generator=g, dtype=torch.int32)
    out = verify_inputs(seed=seed, device=device, with_prev=ragged, **cfg)
    out["seed"] = SAMPLE_SEED + seed_off
    out["name"] = name
    return out


def markov_inputs(R, gamma, V, rank, H, rank_e, sigma_u=2.0, sigma_f=0.02, seed=BASE_SEED + 4,
                  device="cpu"):
    """Inputs of the Markov drafting head: U [R][gamma][V], A and Ct
    [gamma][V][rank], h [R][gamma][H], E [V][rank_e] (all bf16), w [H+rank_e]
    fp32, x0 [R] int32."""
    g = _gen(device, seed)
    bf = torch.bfloat16
    U = _normal((R, gamma, V), sigma_u, g, device).to(bf)
    A = torch.empty((gamma, V, rank), dtype=bf, device=device)
    Ct = torch.empty((gamma, V, rank), dtype=bf, device=device)
    for k in range(gamma):
        A[k] = _normal((V, rank), sigma_f, g, device).to(bf)
        Ct[k] = _normal((V, rank), sigma_f, g, device).to(bf)
    h = _normal((R, gamma, H), 1.0, g, device).to(bf)
    E = _normal((V, rank_e), sigma_f, g, device).to(bf)
    w = _normal((H + rank_e,), sigma_f, g, device)
    x0 = torch.randint(0, V, (R,), generator=g, device=device, dtype=torch.int32)
    return dict(R=R, gamma=gamma, V=V, rank=rank, H=H, rank_e=rank_e, U=U, A=A, Ct=Ct, h=h,
                E=E, w=w, x0=x0, temperature=1.0, seed=SAMPLE_SEED + 4, pos0=None)


def markov_config(device="cpu", **over):
    cfg = dict(MARKOV)
    cfg.pop("sps")
    seed_off = cfg.pop("seed_off")
    cfg.update(over)
    return markov_inputs(seed=BASE_SEED + seed_off, device=device, **cfg)


def rnn_inputs(R, gamma, V, d, H, rank_e, sigma_u=2.0, sigma_w=0.5, sigma_e=1.0, sigma_c=0.05,
               sigma_f=0.02, seed=BASE_SEED + 5, device="cpu"):
    """Inputs of the RNN drafting head: U [R][gamma][V], W [d][d] with entries
    N(0, (sigma_w / sqrt(d))^2) (spectral radius about sigma_w), E_s [V][d]
    N(0, sigma_e^2), Ct [V][d] N(0, sigma_c^2) (row v is column v of C), and
    the confidence head's h, E, w as for the Markov head; all bf16 but w."""
    g = _gen(device, seed)
    bf = torch.bfloat16
    U = _normal((R, gamma, V), sigma_u, g, device).to(bf)
    W = _normal((d, d), sigma_w / math.sqrt(d), g, device).to(bf)
    Es = _normal((V, d), sigma_e, g, device).to(bf)
    Ct = _normal((V, d), sigma_c, g, device).to(bf)
    h = _normal((R, gamma, H), 1.0, g, device).to(bf)
    E = _normal((V, rank_e), sigma_f, g, device).to(bf)
    w = _normal((H + rank_e,), sigma_f, g, device)
    x0 = torch.randint(0, V, (R,), generator=g, device=device, dtype=torch.int32)
    return dict(R=R, gamma=gamma, V=V, d=d, H=H, rank_e=rank_e, U=U, W=W, Es=Es, Ct=Ct, h=h, E=E,
                w=w, x0=x0, temperature=1.0, seed=SAMPLE_SEED + 5, pos0=None)


def rnn_config(device="cpu", **over):
    cfg = dict(RNN)
    seed_off = cfg.pop("seed_off")
    cfg.update(over)
    return rnn_inputs(seed=BASE_SEED + seed_off, device=device, **cfg)


def markov_targets(U, seed=BASE_SEED + 40, sigma=1.5, sigma_bonus=2.0):
    """Target rows for verifying a drafted block, from the seeded backbone
    logits U [R][gamma][V] (the drafted rows are U plus a small bias): the row
    of position k is U_k plus N(0, 1.5^2); the bonus row is N(0, 2^2).
    Returns tgt [R*(gamma+1)][V] bf16 in the reserved-slot layout."""
    R, gamma, V = U.shape
    device = U.device
    g = _gen(device, seed)
    tgt = torch.empty((R, gamma + 1, V), dtype=torch.bfloat16, device=device)
    for r0 in range(0, R, 16):
        r1 = min(R, r0 + 16)
        tgt[r0:r1, :gamma] = (U[r0:r1].float()
                              + _normal((r1 - r0, gamma, V), sigma, g, device)).to(torch.bfloat16)
        tgt[r0:r1, gamma] = _normal((r1 - r0, V), sigma_bonus, g, device).to(torch.bfloat16)
    b_sat, amp, period = MARKOV["sps"]
    sps = sps_table(R * (gamma + 1), b_sat, amp, period).to(device)
    return tgt.view(R * (gamma + 1), V), sps


def headline_bytes(R, gmax, V, esize=2):
    """Algorithmic bytes of one full-block verify: every target and draft row once."""
    return esize * V * (R * (gmax + 1) + R * gmax)


assert math.isclose(headline_bytes(256, 11, 151936) / 1e9, 1.789, rel_tol=1e-3)
