"""GPU parity of the device quota controller lrm_quota_waterfill_device with
the quota oracle (integer quotas, compared exactly), and the controller and
the pruned backward on one stream: device quotas straight into the fused call
(LRM_QUOTA_ON_DEVICE), captured in one HIP graph at any expert count."""

import numpy as np
import pytest
import torch

from oracle import quota as Q
from pruned_expert_backward_lrm_amd import synth

from parity import judge_linear, judge_swiglu, run_linear, run_swiglu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from pruned_expert_backward_lrm_amd import lrm
    return lrm


def say(*a):
    print(*a, flush=True)


def _device_quota(L, pairs, E, budget, counts=None):
    q = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    c = None if counts is None else torch.as_tensor(np.asarray(counts, np.int32), device=DEV)
    ws = L.lrm_quota_waterfill_device(pairs, budget, q, counts=c)
    torch.cuda.synchronize()
    return q.cpu().numpy(), ws


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_workload_counts_match_oracle(L, cfg):
    """The workloads' own routings: counts from the pairs (computed on the
    device) and counts passed in, at several budgets from 0 to beyond N."""
    spec = synth.CONFIGS[cfg]
    r = synth.make_routing(spec["T"], spec["E"], spec["k"], spec["zipf"], "cfg", cfg,
                           local=spec.get("local"))
    pairs = L.Pairs.from_routing(r, DEV)
    for frac in (0.0, 0.05, 0.19, 0.5, 0.9, 1.0, 3.0):
        B = int(frac * r.N) + (cfg if frac else 0)
        want = Q.waterfill(r.counts, B)
        got, ws = _device_quota(L, pairs, r.E, B)
        assert got.tolist() == want.tolist(), (cfg, B)
        assert L.lrm_check_device_errors(ws) == 0
        got2, _ = _device_quota(L, pairs, r.E, B, counts=r.counts)
        assert got2.tolist() == want.tolist(), (cfg, B, "given counts")
    say(f"config {cfg}: quotas equal to the oracle at 7 budgets")


@pytest.mark.parametrize("seed", range(2))
def test_random_counts_match_oracle(L, seed):
    """Random skewed counts, 1..4096 experts (the largest E the library takes)."""
    rng = np.random.default_rng([43, seed])
    none_i = torch.zeros(0, dtype=torch.int32, device=DEV)
    for E in (1, 7, 128, 1000, 4096):
        # the controller takes E from the pairs; the counts are given
        pairs = L.Pairs(none_i, none_i, torch.zeros(0, device=DEV), 0, E)
        for _ in range(4):
            n = (rng.zipf(1.3, E).clip(max=200000) - 1).astype(np.int32)
            B = int(rng.integers(0, int(n.sum()) + 10))
            got, _ = _device_quota(L, pairs, E, B, counts=n)
            assert got.tolist() == Q.waterfill(n, B).tolist(), (E, B)


def test_pairs_out_of_range_are_not_counted(L):
    r = synth.make_routing(64, 6, 2, 0.5, "quota", 9)
    r.expert = r.expert.copy()
    r.expert[3] = r.E + 2
    pairs = L.Pairs.from_routing(r, DEV)
    good = np.bincount(r.expert[r.expert < r.E], minlength=r.E)
    got, ws = _device_quota(L, pairs, r.E, 40)
    assert got.tolist() == Q.waterfill(good, 40).tolist()
    assert L.lrm_check_device_errors(ws) == L.LRM_ERR_INDEX


def test_controller_then_linear_backward(L):
    """Controller and backward on one stream: the device quotas give the same
    kept sets and bit-identical gradients as the host controller's quotas
    passed from the host, and meet the oracle."""
    p = synth.make_config(2, device=DEV)
    r = p["routing"]
    B = int(0.19 * r.N)
    host_q = L.lrm_quota_waterfill(r.counts, B)
    pairs = L.Pairs.from_routing(r, DEV)
    dq, _ = _device_quota(L, pairs, r.E, B)
    assert dq.tolist() == host_q.tolist()
    ph = dict(p, quota=host_q)
    qd = torch.as_tensor(host_q, device=DEV)
    pd = dict(p, quota=qd)
    a = run_linear(L, ph, DEV)
    b = run_linear(L, pd, DEV, flags=L.LRM_QUOTA_ON_DEVICE)
    for k in ("dW", "dX", "pos", "offsets"):
        assert torch.equal(a[k], b[k]), k
    host = dict(ph, X=p["X"].cpu(), G=p["G"].cpu(), W=p["W"].cpu())
    s = judge_linear(host, a)
    say("config 2 under the controller's quotas", s)


def test_controller_then_swiglu_backward(L):
    """SwiGLU with the controller's quotas for all three projections, read on
    the device; judged against the oracle."""
    p = synth.make_swiglu(900, 16, 4, 256, 136, dtype="bf16", seed=23, zipf=1.4, g_std=1e-2)
    r = p["routing"]
    B = int(0.4 * r.N)
    pairs = L.Pairs.from_routing(r, DEV)
    dq, _ = _device_quota(L, pairs, r.E, B)
    assert dq.tolist() == Q.waterfill(r.counts, B).tolist()
    q = torch.as_tensor(dq, device=DEV)
    pd = dict(p, quota_down=q, quota_gate=q, quota_up=q)
    res = run_swiglu(L, pd, DEV, flags=L.LRM_QUOTA_ON_DEVICE)
    ph = dict(p, quota_down=dq, quota_gate=dq.copy(), quota_up=dq.copy())
    s = judge_swiglu(ph, res)
    say("swiglu under the controller's quotas", s)


def test_controller_and_backward_in_one_graph(L):
    """Controller plus backward captured together at E = 600 (beyond the 512
    experts whose host quotas travel in the kernel arguments) and replayed with
    eager work in between: every replay equals the eager pair of calls."""
    p = synth.make_linear(1500, 600, 2, 64, 64, dtype="bf16", seed=33, zipf=1.1)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    X, G, W = (p[k].to(DEV) for k in ("X", "G", "W"))
    q = torch.zeros(r.E, dtype=torch.int32, device=DEV)
    pb = L.linear_problem(pairs, X, "token", G, "pair", W, q, L.LRM_QUOTA_ON_DEVICE)
    out = dict(dW=torch.empty(r.E, 64, 64, device=DEV), dX=torch.empty(r.T, 64, device=DEV),
               pos=torch.empty(r.N, dtype=torch.int32, device=DEV),
               offsets=torch.empty(r.E + 1, dtype=torch.int32, device=DEV))
    ws = torch.empty(L.lrm_workspace_size(pb), dtype=torch.uint8, device=DEV)
    B = r.N // 3
    qws = L.lrm_quota_waterfill_device(pairs, B, q)  # its workspace, allocated outside

    def both():
        L.lrm_quota_waterfill_device(pairs, B, q, ws=qws)
        L.lrm_expert_backward(pb, out, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        both()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = {k: v.cpu().clone() for k, v in out.items()}
    assert q.cpu().tolist() == Q.waterfill(r.counts, B).tolist()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        both()
    for _ in range(3):
        for v in list(out.values()) + [q]:
            v.fill_(-7) if v.dtype == torch.int32 else v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v.cpu(), eager[k]), k
