"""GPU parity of lrm_receiver_layout (the receiver-major layout of the packed
rows for a replica assignment) with the oracle's receiver_layout: every
output is an integer and must match bit for bit."""

import numpy as np
import pytest
import torch

from oracle import redistribute as R
from pruned_expert_backward_lrm_amd import lrm as L
from pruned_expert_backward_lrm_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layout(Me, x, max_rows=None):
    offsets = np.concatenate([[0], np.cumsum(Me)]).astype(np.int32)
    M = int(offsets[-1])
    cap = M if max_rows is None else max_rows
    print(f"layout E={len(Me)} G={x.shape[1]} M={M} max_rows={cap}", flush=True)
    so, bo, dst, ws = L.lrm_receiver_layout(torch.as_tensor(offsets, device=DEV),
                                            torch.as_tensor(np.ascontiguousarray(x, np.int32),
                                                            device=DEV), cap)
    assert L.lrm_check_device_errors(ws) == 0
    ref = R.receiver_layout(offsets, x)
    assert so.cpu().numpy().tolist() == ref[0].tolist()
    assert bo.cpu().numpy().tolist() == ref[1].tolist()
    got = dst.cpu().numpy()
    assert got[:min(M, cap)].tolist() == ref[2][:min(M, cap)].tolist()
    return got


@pytest.mark.parametrize("seed", range(4))
def test_layout_random_matches_oracle(seed):
    rng = np.random.default_rng([505, seed])
    for _ in range(6):
        E, G = int(rng.integers(1, 200)), int(rng.integers(1, 17))
        Me = rng.integers(0, 300, E)
        Me[rng.random(E) < 0.2] = 0
        Rm = rng.random((E, G)) < 0.3
        Rm[np.arange(E), rng.integers(0, G, E)] = True
        _, x = L.lrm_redistribute(Me, Rm)
        _layout(Me, x)


def test_layout_edges():
    _layout(np.array([5, 0, 7]), np.array([[5], [0], [7]]))          # one receiver: identity
    _layout(np.array([0, 0]), np.zeros((2, 3), np.int64))             # nothing kept
    _layout(np.array([3, 3]), np.array([[2, 1], [1, 2]]))             # the hand example
    got = _layout(np.array([4, 2]), np.array([[1, 3], [2, 0]]), max_rows=10)
    assert got[:6].tolist() == R.receiver_layout([0, 4, 6], [[1, 3], [2, 0]])[2].tolist()
    _layout(np.array([9, 1, 5]), np.array([[2, 3, 4], [0, 1, 0], [5, 0, 0]]), max_rows=7)
    E = 4096  # the largest expert count
    Me = np.random.default_rng(1).integers(0, 4, E)
    x = np.zeros((E, 2), np.int64)
    x[:, 0] = Me // 2
    x[:, 1] = Me - Me // 2
    _layout(Me, x)


def test_layout_flags_a_mismatched_assignment():
    offsets = torch.tensor([0, 3, 5], dtype=torch.int32, device=DEV)
    bad = torch.tensor([[2, 0], [1, 1]], dtype=torch.int32, device=DEV)  # expert 0 sums to 2, not 3
    print("layout with a mismatched assignment", flush=True)
    _, _, _, ws = L.lrm_receiver_layout(offsets, bad, 5)
    assert L.lrm_check_device_errors(ws) == L.LRM_ERR_INDEX
    assert L.lrm_check_device_errors(ws) == 0  # cleared
    neg = torch.tensor([[4, -1], [1, 1]], dtype=torch.int32, device=DEV)
    _, _, _, ws = L.lrm_receiver_layout(offsets, neg, 5)
    assert L.lrm_check_device_errors(ws) == L.LRM_ERR_INDEX


def test_layout_after_selection():
    """The selection of the Qwen3-30B-A3B-shaped projection (config 2) over
    8 GPUs, each expert owned by one, the 16 most loaded replicated on all:
    select on the GPU, solve on the host, lay out on the GPU."""
    p = synth.make_config(2, device=DEV)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    X, G = L.mat(p["X"], "token"), L.mat(p["G"], "pair")
    score = torch.empty(r.N, dtype=torch.float32, device=DEV)
    L.lrm_score(pairs, X, G, score)
    i32 = dict(dtype=torch.int32, device=DEV)
    pos, kept, offsets = torch.empty(r.N, **i32), torch.empty(r.N, **i32), torch.empty(r.E + 1, **i32)
    L.lrm_select(pairs, score, p["quota"], pos, offsets, kept, device=DEV)
    Me = np.diff(offsets.cpu().numpy().astype(np.int64))
    Rm = np.zeros((r.E, 8), bool)
    Rm[np.arange(r.E), np.arange(r.E) % 8] = True
    Rm[np.argsort(-Me)[:16]] = True
    peak, x = L.lrm_redistribute(Me, Rm)
    assert peak == R.min_peak(Me, Rm)[0]
    _layout(Me, x)
