"""Pins of the redistribution oracle (oracle/redistribute.py) against things
other than itself: hand-worked fixtures (tests/golden/hand_redistribute.json),
brute-force enumeration of every assignment on tiny cases, the cut (Hall)
condition computed without any flow, and closed forms (a single replica per
expert, full replication, one GPU)."""

import json
import os

import numpy as np
import pytest

from oracle import redistribute as R

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_redistribute.json")


def _case(c):
    return (np.array(c["M"]), np.array(c["R"], bool),
            None if c["base"] is None else np.array(c["base"]),
            None if c["cap"] is None else np.array(c["cap"]))


def test_golden_peaks_and_unique_assignments():
    d = json.load(open(GOLD))
    for c in d["cases"]:
        M, Rm, base, cap = _case(c)
        peak, x = R.min_peak(M, Rm, base, cap)
        assert peak == c["peak"], c["why"]
        assert R.check_assignment(M, Rm, x, base, cap) == c["peak"], c["why"]
        if c["x"] is not None:
            assert x.tolist() == c["x"], c["why"]


def test_golden_receiver_layout():
    lay = json.load(open(GOLD))["layout"]
    send_off, blk_off, dst = R.receiver_layout(lay["offsets"], lay["x"])
    assert send_off.tolist() == lay["send_off"]
    assert blk_off.tolist() == lay["blk_off"]
    assert dst.tolist() == lay["dst"]


def _random_case(rng, E, G, mmax, with_base, with_cap):
    M = rng.integers(0, mmax + 1, E)
    Rm = rng.random((E, G)) < 0.5
    for e in range(E):
        if not Rm[e].any():
            Rm[e, rng.integers(G)] = True
    base = rng.integers(0, 4, G) if with_base else None
    cap = rng.integers(1, mmax * E + 1, G) if with_cap else None
    return M, Rm, base, cap


@pytest.mark.parametrize("seed", range(6))
def test_flow_equals_brute_force_and_cut_bound(seed):
    rng = np.random.default_rng([77, seed])
    n = 0
    while n < 60:
        E, G = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        M, Rm, base, cap = _random_case(rng, E, G, 4, seed % 2 == 1, seed % 3 == 2)
        try:
            bf = R.brute_force_peak(M, Rm, base, cap)
        except R.Infeasible:
            with pytest.raises(R.Infeasible):
                R.min_peak(M, Rm, base, cap)
            continue
        peak, x = R.min_peak(M, Rm, base, cap)
        assert peak == bf
        assert R.check_assignment(M, Rm, x, base, cap) == bf
        assert R.hall_peak(M, Rm, base, cap) == bf
        n += 1


def test_single_replica_is_fixed_ownership():
    rng = np.random.default_rng(5)
    E, G = 12, 4
    M = rng.integers(0, 50, E)
    owner = rng.integers(0, G, E)
    Rm = np.zeros((E, G), bool)
    Rm[np.arange(E), owner] = True
    base = rng.integers(0, 10, G)
    peak, x = R.min_peak(M, Rm, base)
    expect = max(base[g] + M[owner == g].sum() for g in range(G))
    assert peak == expect
    assert (x[np.arange(E), owner] == M).all()


@pytest.mark.parametrize("E,G", [(5, 3), (16, 8), (7, 1)])
def test_full_replication_is_balanced(E, G):
    M = np.random.default_rng([E, G]).integers(0, 40, E)
    peak, x = R.min_peak(M, np.ones((E, G), bool))
    assert peak == -(-int(M.sum()) // G)
    assert R.check_assignment(M, np.ones((E, G), bool), x) == peak


def test_infeasible_cases_raise():
    with pytest.raises(R.Infeasible):
        R.min_peak([3, 1], np.array([[1, 0], [0, 0]], bool))
    with pytest.raises(R.Infeasible):
        R.min_peak([3, 4], np.array([[1, 0], [1, 0]], bool), cap=[6, 10])
    # no kept pairs on an expert without replicas is fine
    assert R.min_peak([0, 2], np.array([[0, 0], [1, 1]], bool))[0] == 1


def test_layout_is_a_block_permutation():
    rng = np.random.default_rng(9)
    E, G = 9, 4
    Me = rng.integers(0, 20, E)
    Rm = rng.random((E, G)) < 0.6
    Rm[np.arange(E), rng.integers(0, G, E)] = True
    _, x = R.min_peak(Me, Rm)
    offsets = np.concatenate([[0], np.cumsum(Me)])
    send_off, blk_off, dst = R.receiver_layout(offsets, x)
    assert sorted(dst.tolist()) == list(range(int(Me.sum())))
    for e in range(E):
        rows = dst[offsets[e]:offsets[e + 1]]
        j = 0
        for g in range(G):
            seg = rows[j:j + x[e, g]]
            start = send_off[g] + blk_off[g, e]
            assert seg.tolist() == list(range(start, start + x[e, g]))
            j += x[e, g]
    one = R.receiver_layout(offsets, Me[:, None])
    assert one[2].tolist() == list(range(int(Me.sum())))
