"""The device counter hash against the oracle's, counter by counter.

Both sides implement SplitMix64 (Steele, Lea, Flood 2014) nested over
(seed, request, position, draw) from its published definition; neither shares
code with the other.  The oracle's hash is pinned to the generator's published
sequence on the CPU; here the device's uniforms (sd_uniforms, the same hash the
verify and drafting kernels draw from) must equal the oracle's bit for bit on
10^6 counters, including request ids and positions past 32 bits and negative
int64 positions (taken as unsigned words)."""

import numpy as np
import pytest
import torch

import draft_verification_amd as sdv
from oracle import rng as ORNG

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("draw", [0, 1, 2])
def test_device_uniforms_equal_the_oracle_on_a_million_counters(draw):
    n = 1_000_000
    g = np.random.default_rng(1000 + draw)
    req = g.integers(0, 1 << 12, n, dtype=np.int64)
    pos = g.integers(0, 1 << 20, n, dtype=np.int64)
    req[: n // 10] = g.integers(-(1 << 62), 1 << 62, n // 10, dtype=np.int64)   # wide request ids
    pos[n // 10: n // 5] = g.integers(-(1 << 62), 1 << 62, n // 10, dtype=np.int64)  # wide positions
    seed = 0xC0FFEE + 3
    out = sdv.sd_uniforms(seed, torch.as_tensor(req, device="cuda"), torch.as_tensor(pos, device="cuda"),
                          draw)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = ORNG.uniforms(seed, req, pos, draw)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} counters differ, first at {bad[:5]}"
    # the scalar (pure-integer) form of the oracle on a subset
    for i in range(0, n, 50_000):
        assert got[i] == ORNG.uniform(seed, int(req[i]), int(pos[i]), draw)
    # 24-bit values in [0, 1 - 2^-24]
    assert got.min() >= 0.0 and got.max() <= 1.0 - 2.0 ** -24
    assert np.all(got * 2 ** 24 == np.floor(got * 2 ** 24))


def test_uniforms_seed_changes_every_value():
    req = torch.arange(4096, dtype=torch.int64, device="cuda")
    pos = torch.full((4096,), 7, dtype=torch.int64, device="cuda")
    a = sdv.sd_uniforms(1, req, pos, 1).cpu().numpy()
    b = sdv.sd_uniforms(2, req, pos, 1).cpu().numpy()
    assert np.mean(a == b) < 0.01
