"""Counter-hash uniforms shared by definition with the GPU path (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages need one uniform per random decision: the rejection-sampling test
and the resampling of a rejected position (speculative-decoding history page,
"1.1 mechanism"), and the sequential draw of each drafted token (DSpark summary,
"innovation one", Markov head).  They fix no generator.  Both sides therefore
implement the same counter-based generator from its published definition:

  SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the 64-bit finaliser with multipliers
  0xbf58476d1ce4e5b9 / 0x94d049bb133111eb and shifts 30/27/31, as used by
  java.util.SplittableRandom).  One step from state x is
  ``mix(x + 0x9e3779b97f4a7c15)``.

Counter layout (a construction of this project, not of the pages)::

    h = sm(sm(sm(sm(seed) ^ r) ^ pos) ^ draw)
    u = (h >> 40) * 2**-24          # 24-bit, exactly representable in fp32

``r`` is the request index, ``pos`` the absolute token position (the caller's
``pos0[r]`` plus the 1-based draft position), ``draw`` the decision kind:
0 = draft sample, 1 = accept test, 2 = correction (residual or bonus) sample.

Pins: the SplitMix64 step against the published reference sequence for seed
1234567, and a chi-square uniformity test (tests/test_oracle_rng.py).  The
nesting itself is a definition, not a result, so it has nothing further to be
pinned against.
"""

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB

DRAW_DRAFT = 0
DRAW_ACCEPT = 1
DRAW_CORRECT = 2


def mix64(z: int) -> int:
    """SplitMix64 output finaliser on a Python int (mod 2**64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MUL1) & MASK64
    z = ((z ^ (z >> 27)) * MUL2) & MASK64
    return z ^ (z >> 31)


def sm(x: int) -> int:
    """One SplitMix64 step taken from state ``x``: mix(x + golden gamma)."""
    return mix64((x + GOLDEN_GAMMA) & MASK64)


def splitmix64_sequence(seed: int, n: int):
    """The generator's first ``n`` outputs from ``seed`` (state advances by gamma)."""
    out = []
    state = seed & MASK64
    for _ in range(n):
        state = (state + GOLDEN_GAMMA) & MASK64
        out.append(mix64(state))
    return out


def counter_hash(seed: int, r: int, pos: int, draw: int) -> int:
    """64-bit hash of the (seed, request, position, draw) counter."""
    h = sm(seed & MASK64)
    h = sm(h ^ (r & MASK64))
    h = sm(h ^ (pos & MASK64))
    return sm(h ^ (draw & MASK64))


def uniform(seed: int, r: int, pos: int, draw: int) -> float:
    """Uniform in [0, 1 - 2**-24] with 24 random bits (a Python float, fp64)."""
    return (counter_hash(seed, r, pos, draw) >> 40) * (2.0 ** -24)


# ---------------------------------------------------------------------------
# Vectorised form: identical arithmetic on numpy uint64 arrays (numpy wraps
# unsigned multiplication mod 2**64).  Used only to draw many counters at once.

def _mix64_np(z):
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MUL1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MUL2)
    return z ^ (z >> np.uint64(31))


def _sm_np(x):
    return _mix64_np(x + np.uint64(GOLDEN_GAMMA))


def uniforms(seed: int, r, pos, draw: int) -> np.ndarray:
    """Vectorised ``uniform`` over broadcast arrays of r and pos (fp64 result)."""
    with np.errstate(over="ignore"):
        r = np.asarray(r).astype(np.int64).astype(np.uint64)
        pos = np.asarray(pos).astype(np.int64).astype(np.uint64)
        h0 = _sm_np(np.uint64(seed & MASK64))
        h = _sm_np(h0 ^ r)
        h = _sm_np(h ^ pos)
        h = _sm_np(h ^ np.uint64(draw & MASK64))
        return (h >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)
