"""Parity of the library's host quota controller lrm_quota_waterfill (no GPU
work) with the quota oracle: integer quotas, compared exactly."""

import numpy as np
import pytest

from oracle import quota as Q
from pruned_expert_backward_lrm_amd import lrm as L
from pruned_expert_backward_lrm_amd import synth


def test_hand_examples():
    for B, expect in ((12, [4, 1, 4, 3]), (13, [5, 1, 4, 3]), (14, [5, 1, 5, 3]),
                      (100, [10, 1, 6, 3]), (0, [0, 0, 0, 0])):
        assert L.lrm_quota_waterfill([10, 1, 6, 3], B).tolist() == expect


@pytest.mark.parametrize("seed", range(3))
def test_random_counts_match_oracle(seed):
    rng = np.random.default_rng([41, seed])
    for _ in range(200):
        E = int(rng.integers(1, 300))
        n = rng.zipf(1.3, E).clip(max=100000) - 1
        B = int(rng.integers(0, n.sum() + 10))
        assert L.lrm_quota_waterfill(n, B).tolist() == Q.waterfill(n, B).tolist()


def test_workload_counts():
    for cfg in (2, 3, 5):
        spec = synth.CONFIGS[cfg]
        r = synth.make_routing(spec["T"], spec["E"], spec["k"], spec["zipf"], "cfg", cfg,
                               local=spec.get("local"))
        for frac in (0.1, 0.19, 0.5, 1.0):
            B = int(frac * r.N)
            assert L.lrm_quota_waterfill(r.counts, B).tolist() == Q.waterfill(r.counts, B).tolist()


def test_errors():
    with pytest.raises(L.LrmError) as ei:
        L.lrm_quota_waterfill([1, -2], 3)
    assert ei.value.status == 6
    with pytest.raises(L.LrmError) as ei:
        L.lrm_quota_waterfill([1, 2], -1)
    assert ei.value.status == 6
