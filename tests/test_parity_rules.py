"""The comparison rules the GPU parity tests apply (tests/parity_util.py),
checked on the CPU: the allowances they grant are bounds that hold, and a
planted error outside them is caught."""

import numpy as np
import pytest

from oracle import verify as OV
from oracle.bf16 import round_to_bf16
from tests.parity_util import (cdf_shift, check_drafted_row_stats, compare_draft_chains, moved_mass,
                               assert_row_stats, NEAR, partings_bound)


def _flip(L, idx):
    """Move the bf16 values at idx by one unit in the last place (up)."""
    out = L.copy()
    for i in idx:
        x = np.float32(out[i])
        bits = np.array([x], np.float32).view(np.uint32)[0]
        step = np.uint32(1 << 16)
        out[i] = np.array([bits + step if x >= 0 else bits - step], np.uint32).view(np.float32)[0]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_cdf_shift_bounds_the_inverse_cdf_difference(seed):
    g = np.random.default_rng(seed)
    V = 2000
    T = float(g.choice([0.5, 1.0, 2.0]))
    L = round_to_bf16(g.normal(0, 3, V))
    L2 = _flip(L, g.choice(V, size=int(g.integers(1, 40)), replace=False))
    p, _, _, _ = OV.row_softmax(L, V, T)
    q, _, _, _ = OV.row_softmax(L2, V, T)
    actual = np.max(np.abs(np.cumsum(p) - np.cumsum(q)))
    bound = cdf_shift(L2, L, V, T)
    assert actual <= bound * (1 + 1e-9) + 1e-15
    assert bound < 1.0


def test_drafted_row_stats_allowance():
    g = np.random.default_rng(7)
    V, T = 3000, 1.0
    L = round_to_bf16(g.normal(0, 2, V))
    L2 = _flip(L, [int(np.argmax(L)), 5, 17])
    _, m2, Z2, _ = OV.row_softmax(L2, V, T)
    check_drafted_row_stats((m2, Z2), L2, L, V, T, "flipped")     # exact stats of the GPU's own row
    with pytest.raises(AssertionError):
        check_drafted_row_stats((m2, Z2 * (1 + 3e-5)), L, L, V, T, "planted")   # identical rows: REL only
    assert moved_mass(L, L, V, T)[0] == 0.0


def test_row_stats_compared_as_normalisers():
    ref = np.array([[3.0, 1.5], [7.0, 2.0]])
    # m rounded up by 4e-6 and Z taken relative to it: the same normaliser
    got = ref.copy()
    got[:, 0] += 4e-6
    got[:, 1] *= np.exp(-4e-6)
    assert_row_stats(got, ref, "shifted m")
    bad = ref.copy()
    bad[:, 1] *= 1 + 2e-5
    with pytest.raises(AssertionError):
        assert_row_stats(bad, ref, "planted Z")


def test_draft_chain_partings():
    ref = dict(tokens=np.array([[1, 2, 3]]), conf=np.array([[0.5, 0.5, 0.5]]),
               dists=np.array([[1.0, 5e-7, 1.0]]))
    conf = np.array([[0.5, 0.5, 0.5]])
    # parting at a near-boundary draw: accepted, the rest not compared
    near, parted, compared, gone = compare_draft_chains(np.array([[1, 9, 7]]), conf, ref, [0])
    assert parted == 1 and compared == 2 and gone == {0}
    # parting at a draw 5e-4 from its boundary: caught ...
    ref5 = dict(ref, dists=np.array([[5e-4, 5e-7, 1.0]]))
    with pytest.raises(AssertionError):
        compare_draft_chains(np.array([[4, 2, 3]]), conf, ref5, [0])
    # ... unless the two rows' inverse CDFs may lie that far apart
    compare_draft_chains(np.array([[4, 2, 3]]), conf, ref5, [0], shift=lambda i, r, k: 8e-4)
    with pytest.raises(AssertionError):   # a bound past 1e-3 means the rows themselves differ
        compare_draft_chains(np.array([[4, 2, 3]]), conf, ref5, [0], shift=lambda i, r, k: 2e-3)
    # a confidence off by more than 1e-5 relative: caught
    with pytest.raises(AssertionError):
        compare_draft_chains(np.array([[1, 2, 3]]), conf * (1 + 3e-5), ref, [0])
    assert NEAR == 1e-6


def test_partings_bound():
    """At most 0.75 % of the positions compared (rounded up, at least one)
    may part, each at a draw the parting rule explains.  At full size the
    heads compare 2025 (Markov) and 1972 (RNN) positions and part at 4 and 8
    of them; the allowance of 16 and 15 stays within twice the observed rate,
    where 2 % (41 and 40) would hide a regression to five times it."""
    assert partings_bound(1) == 1
    assert partings_bound(20) == 1
    assert partings_bound(134) == 2
    assert partings_bound(2025) == 16
    assert partings_bound(1972) == 15
    for compared in (50, 260, 1000, 2025, 4096):
        b = partings_bound(compared)
        assert b >= 1 and b <= max(1, 0.0075 * compared + 1)

