"""Pins of the quota-controller oracle (oracle/quota.py): brute-force
min-max over every quota vector on tiny cases, closed forms (budget above the
total keeps everything, equal counts split evenly, budget zero keeps nothing)
and the structural properties of water-filling caps."""

import numpy as np
import pytest

from oracle import quota as Q


def _props(n, B, q):
    n = np.asarray(n)
    assert (q >= 0).all() and (q <= n).all()
    assert q.sum() == min(B, n.sum())
    cut = q < n
    if cut.any():
        top = q.max()
        assert q[cut].min() >= top - 1  # a cut expert keeps the cap, or the cap minus one
        # among cut experts, those keeping the cap come first (the extra pairs
        # of the budget go to the lowest indices)
        c = np.nonzero(cut)[0]
        at_top = q[c] == top
        if at_top.any() and (~at_top).any():
            assert c[at_top].max() < c[~at_top].min()


def test_hand_examples():
    # counts 10, 1, 6, 3 with budget 12: tau = 4 keeps 4+1+4+3 = 12
    assert Q.waterfill([10, 1, 6, 3], 12).tolist() == [4, 1, 4, 3]
    # budget 13: tau = 4 leaves one pair, to the first expert above the cap (expert 0)
    assert Q.waterfill([10, 1, 6, 3], 13).tolist() == [5, 1, 4, 3]
    # budget 14: two extra pairs, to experts 0 and 2
    assert Q.waterfill([10, 1, 6, 3], 14).tolist() == [5, 1, 5, 3]
    assert Q.waterfill([10, 1, 6, 3], 100).tolist() == [10, 1, 6, 3]
    assert Q.waterfill([10, 1, 6, 3], 0).tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("seed", range(4))
def test_min_max_equals_brute_force(seed):
    rng = np.random.default_rng([31, seed])
    for _ in range(120):
        E = int(rng.integers(1, 5))
        n = rng.integers(0, 6, E)
        B = int(rng.integers(0, n.sum() + 3))
        q = Q.waterfill(n, B)
        assert q.max(initial=0) == Q.brute_force_min_max(n, B)
        _props(n, B, q)


def test_equal_counts_split_evenly():
    q = Q.waterfill([50] * 8, 100)
    assert q.tolist() == [13, 13, 13, 13, 12, 12, 12, 12]


def test_large_random_properties():
    rng = np.random.default_rng(8)
    for _ in range(50):
        n = rng.zipf(1.5, 128).clip(max=20000)
        B = int(rng.integers(0, n.sum() + 1))
        _props(n, B, Q.waterfill(n, B))
