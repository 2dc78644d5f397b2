"""bfloat16 round-to-nearest-even, written from the format's definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and fp32's 8-bit
exponent range.  Rounding a real x to bf16 means rounding it to the nearest
multiple of its quantum, ties to the even multiple, where the quantum is
2**(e - 8) for x = m * 2**e with m in [0.5, 1) (normal range) and 2**-133 below
the smallest normal 2**-126.  Overflow past the largest finite bf16 gives inf.

The Markov head's drafted logits are rounded to bf16 before they are sampled
from and handed to verification (DSpark summary, "innovation one"; the rounding
itself is this project's reading: the distribution that was sampled must be the
one the verifier sees).

Pin: agreement with torch's fp32->bf16 conversion on fp32-exact inputs
(tests/test_oracle_pins.py).
"""

import numpy as np

_BF16_MAX = float.fromhex("0x1.fep127")


def round_to_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even); fp64 result."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    _, e = np.frexp(xf)
    e = np.maximum(e, -125)
    quantum = np.ldexp(np.ones_like(xf), e - 8)
    y = np.rint(xf / quantum) * quantum  # np.rint rounds half to even
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, y), y)
    out[finite] = y
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to fp64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Encode values that are already bf16-representable as raw uint16 bits."""
    y = np.asarray(x, dtype=np.float64).astype(np.float32)
    b = y.view(np.uint32)
    if np.any((b & np.uint32(0xFFFF)) != 0):
        raise ValueError("value is not representable in bf16")
    return (b >> np.uint32(16)).astype(np.uint16)
