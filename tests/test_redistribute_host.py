"""Parity of the library's host solver lrm_redistribute (a host function of
the C ABI: no GPU work) with the redistribution oracle: the optimal peak is
unique and must match exactly; the assignment, which in general is not
unique, must be valid and reach that peak."""

import json
import os

import numpy as np
import pytest

from oracle import redistribute as R
from pruned_expert_backward_lrm_amd import lrm as L
from pruned_expert_backward_lrm_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_redistribute.json")


def test_golden_cases():
    for c in json.load(open(GOLD))["cases"]:
        Rm = np.array(c["R"], bool)
        peak, x = L.lrm_redistribute(c["M"], Rm, c["base"], c["cap"])
        assert peak == c["peak"], c["why"]
        assert R.check_assignment(c["M"], Rm, x, c["base"], c["cap"]) == peak
        if c["x"] is not None:
            assert x.tolist() == c["x"], c["why"]


@pytest.mark.parametrize("seed", range(4))
def test_random_cases_match_oracle(seed):
    rng = np.random.default_rng([404, seed])
    for it in range(80):
        E, G = int(rng.integers(1, 48)), int(rng.integers(1, 10))
        M = rng.integers(0, 80, E)
        Rm = rng.random((E, G)) < 0.35
        Rm[np.arange(E), rng.integers(0, G, E)] = True
        if it % 7 == 0:
            Rm[rng.integers(E)] = False  # an expert without replicas
        base = rng.integers(0, 40, G) if it % 2 else None
        cap = rng.integers(10, 600, G) if it % 3 == 0 else None
        try:
            po, _ = R.min_peak(M, Rm, base, cap)
        except R.Infeasible:
            with pytest.raises(L.LrmError) as ei:
                L.lrm_redistribute(M, Rm, base, cap)
            assert ei.value.status == L.LRM_ERR_INFEASIBLE
            continue
        pn, xn = L.lrm_redistribute(M, Rm, base, cap)
        assert pn == po
        assert R.check_assignment(M, Rm, xn, base, cap) == po


def test_tiny_cases_match_brute_force():
    rng = np.random.default_rng(11)
    for _ in range(150):
        E, G = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        M = rng.integers(0, 5, E)
        Rm = rng.random((E, G)) < 0.5
        Rm[np.arange(E), rng.integers(0, G, E)] = True
        cap = rng.integers(0, 8, G) if rng.random() < 0.3 else None
        try:
            bf = R.brute_force_peak(M, Rm, None, cap)
        except R.Infeasible:
            continue
        assert L.lrm_redistribute(M, Rm, None, cap)[0] == bf


def test_expert_parallel_shape():
    """The Qwen3-30B-A3B-shaped selection (128 experts) spread over 8 GPUs:
    each expert owned by one GPU, the 16 most loaded replicated everywhere."""
    spec = synth.CONFIGS[2]
    r = synth.make_routing(spec["T"], spec["E"], spec["k"], spec["zipf"], "cfg", 2)
    Me = np.minimum(synth._quotas(2, r, None)["quota"], r.counts)
    E, G = r.E, 8
    Rm = np.zeros((E, G), bool)
    Rm[np.arange(E), np.arange(E) % G] = True
    Rm[np.argsort(-Me)[:16]] = True
    peak, x = L.lrm_redistribute(Me, Rm)
    assert peak == R.min_peak(Me, Rm)[0] == R.hall_peak(Me, Rm)
    assert R.check_assignment(Me, Rm, x) == peak
    fixed = max(Me[np.arange(E) % G == g].sum() for g in range(G))
    assert peak <= fixed


def test_argument_errors():
    with pytest.raises(L.LrmError) as ei:
        L.lrm_redistribute([1, -1], np.ones((2, 2), bool))
    assert ei.value.status == 6  # LRM_ERR_QUOTA
    with pytest.raises(L.LrmError) as ei:
        L.lrm_redistribute([1, 1], np.ones((2, 2), bool), base=[0, -3])
    assert ei.value.status == 2  # LRM_ERR_SHAPE
    peak, x = L.lrm_redistribute([0, 0], np.zeros((2, 3), bool))  # nothing kept, no replicas
    assert peak == 0 and not x.any()
