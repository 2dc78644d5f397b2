"""Pins for the oracle's bf16 rounding against torch's fp32->bf16 conversion."""

import numpy as np
import torch

from oracle.bf16 import round_to_bf16, bf16_bits_to_f64, f64_to_bf16_bits


def test_round_to_bf16_matches_torch_on_fp32_inputs():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.normal(0, 3, 200000),
        g.normal(0, 1e-30, 1000),
        g.normal(0, 1e-39, 1000),                 # bf16 subnormal range
        g.normal(0, 1e30, 1000),
    ]).astype(np.float32)
    # exact ties: low 16 bits = 0x8000
    ties = (g.integers(0, 2**31, 5000, dtype=np.int64).astype(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    ties = ties.view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bits_roundtrip():
    g = np.random.default_rng(1)
    x = round_to_bf16(g.normal(0, 5, 1000))
    assert np.array_equal(bf16_bits_to_f64(f64_to_bf16_bits(x)), x)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(t.view(torch.int16).numpy().view(np.uint16), f64_to_bf16_bits(x))
