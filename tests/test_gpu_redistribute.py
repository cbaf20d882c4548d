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


def test_compaction_into_receiver_blocks():
    """The config-2 selection spread over 8 GPUs (experts owned round robin,
    the 16 most loaded replicated on all), then compaction straight into the
    receiver-major blocks: the row map matches the oracle's receiver layout
    bit for bit, every receiver-major row is the expert-major packed row it
    maps from (bit for bit), and equals the fp64 w x (or g) row of the pair
    packed there, within one bf16 rounding (exactly for g)."""
    from oracle import lrm_oracle as O
    p = synth.make_config(2, device=DEV)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    X, G = L.mat(p["X"], "token"), L.mat(p["G"], "pair")
    score = torch.empty(r.N, dtype=torch.float32, device=DEV)
    L.lrm_score(pairs, X, G, score)
    i32 = dict(dtype=torch.int32, device=DEV)
    pos, kept, offsets = torch.empty(r.N, **i32), torch.empty(r.N, **i32), torch.empty(r.E + 1, **i32)
    L.lrm_select(pairs, score, p["quota"], pos, offsets, kept, device=DEV)
    offs = offsets.cpu().numpy().astype(np.int64)
    Me = np.diff(offs)
    M = int(offs[-1])
    Rm = np.zeros((r.E, 8), bool)
    Rm[np.arange(r.E), np.arange(r.E) % 8] = True
    Rm[np.argsort(-Me, kind="stable")[:16]] = True
    _, x = L.lrm_redistribute(Me, Rm)
    dst = torch.as_tensor(_layout(Me, x), device=DEV)
    di, do = p["d_in"], p["d_out"]
    bf = dict(dtype=torch.bfloat16, device=DEV)
    Xp, Gp = torch.zeros(M, di, **bf), torch.zeros(M, do, **bf)
    Xr, Gr = torch.zeros(M, di, **bf), torch.zeros(M, do, **bf)
    L.lrm_compact(pairs, kept, offsets, M, X, G, Xp, Gp)
    L.lrm_compact_rows(pairs, kept, offsets, M, dst, X, G, Xr, Gr)
    torch.cuda.synchronize()
    d = dst.long()
    assert torch.equal(Xr[d], Xp) and torch.equal(Gr[d], Gp)
    # against the oracle: its row map for these kept counts, and the fp64 rows
    # of the pairs packed there (the kept sets themselves are judged by the
    # selection parity tests)
    host = dict(p, X=p["X"].cpu(), G=p["G"].cpu())
    _, _, odst = R.receiver_layout(offs, x)
    assert odst.tolist() == dst.cpu().numpy().tolist()
    ids = kept[:M].cpu().numpy().astype(np.int64)
    inv = np.empty(M, np.int64)
    inv[odst] = np.arange(M)
    ids_at = ids[inv]  # pair packed at each receiver-major row
    g64 = O.pair_rows(host["G"], "pair", r.token, ids_at)
    x64 = O.pair_rows(host["X"], "token", r.token, ids_at) * r.weight[ids_at][:, None]
    assert np.array_equal(Gr.double().cpu().numpy(), g64)
    rel = np.abs(Xr.double().cpu().numpy() - x64) / np.maximum(np.abs(x64), 1e-30)
    assert rel.max() <= 2.0 ** -8, rel.max()
