"""GPU parity of the single-projection (LINEAR) pruned backward, through the C
ABI, against the fp64 oracle: each step on its own, then the fused call."""

import numpy as np
import pytest
import torch

from oracle import lrm_oracle as O
from pruned_expert_backward_lrm_amd import synth

from parity import (TOL, check_packing, check_selection, judge_linear, kept_from_pos, rel_fro,
                    run_linear)

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


# ----------------------------------------------------------------- score

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("x_rows,g_rows", [("token", "pair"), ("pair", "token"),
                                           ("token", "token"), ("pair", "pair")])
def test_score_layouts(L, dtype, x_rows, g_rows):
    say("score", dtype, x_rows, g_rows)
    p = synth.make_linear(300, 6, 3, 72 if dtype == "f32" else 80, 48, dtype=dtype,
                          x_rows=x_rows, g_rows=g_rows, seed=1)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    X, G = p["X"].to(DEV), p["G"].to(DEV)
    score = torch.empty(r.N, device=DEV)
    L.lrm_score(pairs, L.mat(X, x_rows), L.mat(G, g_rows), score)
    torch.cuda.synchronize()
    np.testing.assert_allclose(score.cpu().numpy().astype(np.float64), O.linear_scores(p),
                               rtol=2 ** -23, atol=0)


def test_score_glu(L):
    say("score_glu")
    p = synth.make_swiglu(200, 5, 2, 64, 96, dtype="bf16", seed=2)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    score = torch.empty(r.N, device=DEV)
    L.lrm_score_glu(pairs, L.mat(p["A"].to(DEV), "pair"), L.mat(p["B"].to(DEV), "pair"),
                    L.mat(p["G"].to(DEV), "token"), score)
    torch.cuda.synchronize()
    # silu in fp32 on the GPU: a few ulp per element, inside the select window
    got = score.cpu().numpy().astype(np.float64)
    ref = O.swiglu_down_scores(p)
    rel = np.abs(got - ref) / ref
    say("  glu score max rel err", rel.max(), "mean", rel.mean())
    assert rel.max() < 1e-6, rel.max()


# ---------------------------------------------------------------- select

def _select(L, r, score_np, quota, flags=0):
    pairs = L.Pairs.from_routing(r, DEV)
    N = max(r.N, 1)
    score = torch.as_tensor(np.asarray(score_np, np.float32), device=DEV)
    pos = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    kept = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((r.E + 1,), -7, dtype=torch.int32, device=DEV)
    ws = L.lrm_select(pairs, score, quota, pos, offsets, kept, flags=flags, device=DEV)
    torch.cuda.synchronize()
    return pos.cpu().numpy()[: r.N], offsets.cpu().numpy(), kept.cpu().numpy(), ws


@pytest.mark.parametrize("case", ["half", "zero", "all", "over", "ones", "ties", "empty_experts",
                                  "single"])
def test_select_cases(L, case):
    say("select", case)
    T, E, k = 700, 9, 2
    p = synth.make_linear(T, E, k, 16, 16, dtype="f32", seed=3, zipf=1.3)
    r = p["routing"]
    rng = np.random.default_rng(4)
    s = rng.random(r.N).astype(np.float32)
    c = r.counts
    q = {"half": c // 2, "zero": 0 * c, "all": c, "over": c + 5, "ones": np.ones_like(c),
         "ties": c // 3, "empty_experts": c // 2, "single": np.minimum(c, 1)}[case]
    if case == "ties":
        s = rng.integers(0, 4, r.N).astype(np.float32)  # massive exact ties
    if case == "empty_experts":
        # experts 0, 3 and 8 receive no pairs at all
        keep = ~np.isin(r.expert, [0, 3, 8])
        r = synth.Routing(r.T, E, k, r.expert[keep], r.token[keep], r.weight[keep],
                          np.bincount(r.expert[keep], minlength=E), {})
        s = s[keep]
        q = r.counts // 2 + (np.arange(E) % 2)
    if case == "single":
        keep = np.zeros(r.N, bool)
        for e in range(E):
            keep[np.nonzero(r.expert == e)[0][:1]] = True
        r = synth.Routing(r.T, E, k, r.expert[keep], r.token[keep], r.weight[keep],
                          np.bincount(r.expert[keep], minlength=E), {})
        s = s[keep]
    pos, offsets, kept, _ = _select(L, r, s, q)
    s64 = s.astype(np.float64)
    ora = O.select_top_quota(r.expert, s64, q, E)
    gk = kept_from_pos(pos, r.expert, E)
    # fp32 keys are the oracle's own inputs here: sets must be identical
    for e in range(E):
        assert np.array_equal(gk[e], ora[e]), f"expert {e}"
    check_packing(pos, offsets, r.expert, E)
    M = offsets[-1]
    assert np.array_equal(kept[:M], np.concatenate(ora) if ora else kept[:0])


def test_select_large_expert(L):
    """One expert with 70k candidates (multi-pass radix, many waves)."""
    say("select large")
    T, E, k = 40000, 4, 2
    rng = np.random.default_rng(5)
    token = np.repeat(np.arange(T, dtype=np.int32), k)
    expert = np.where(rng.random(T * k) < 0.88, 0, rng.integers(1, E, T * k)).astype(np.int32)
    r = synth.Routing(T, E, k, expert, token, rng.random(T * k).astype(np.float32),
                      np.bincount(expert, minlength=E), {})
    s = (rng.standard_normal(r.N) ** 2 * 1e-3).astype(np.float32)
    s[::97] = s[5]  # ties straddling the threshold region
    q = (r.counts * 3) // 7
    pos, offsets, kept, _ = _select(L, r, s, q)
    ora = O.select_top_quota(r.expert, s.astype(np.float64), q, E)
    gk = kept_from_pos(pos, r.expert, E)
    for e in range(E):
        assert np.array_equal(gk[e], ora[e]), f"expert {e}"
    check_packing(pos, offsets, r.expert, E)


def test_select_bucket_rows_ragged(L):
    """A histogram of 100 experts x 391 blocks (100000 pairs): at least 32768
    counts, so its rows are scanned by many workgroups (one wave per expert,
    a partial last workgroup, rows not a multiple of 64 blocks) before the
    offsets are formed.  Kept sets against the oracle, ties included, and
    one expert with no pair at all."""
    say("select, many-workgroup histogram rows")
    T, E, k = 50000, 100, 2
    rng = np.random.default_rng(17)
    token = np.repeat(np.arange(T, dtype=np.int32), k)
    expert = rng.integers(0, E - 1, T * k).astype(np.int32)  # expert E - 1 gets none
    r = synth.Routing(T, E, k, expert, token, rng.random(T * k).astype(np.float32),
                      np.bincount(expert, minlength=E), {})
    s = (rng.standard_normal(r.N) ** 2 * 1e-3).astype(np.float32)
    s[::53] = s[7]
    q = (r.counts * 5) // 9 + (np.arange(E) % 3 == 0)
    pos, offsets, kept, _ = _select(L, r, s, q)
    ora = O.select_top_quota(r.expert, s.astype(np.float64), q, E)
    gk = kept_from_pos(pos, r.expert, E)
    for e in range(E):
        assert np.array_equal(gk[e], ora[e]), f"expert {e}"
    check_packing(pos, offsets, r.expert, E)


@pytest.mark.parametrize("case", ["tiny_fp32", "ties_8192", "wide_1024", "device_quota",
                                  "bad_indices"])
def test_select_one_launch_matches_bucketing(L, case, monkeypatch):
    """The one-launch selection of small calls (one workgroup per expert that
    histograms every pair itself) against the bucketing kernels followed by
    the per-expert select (LRM_SELECT_ONE_LAUNCH=0): pos, kept offsets, the
    kept list and the error word bit for bit.  Cases: the tiny fp32 workload's
    routing and quotas; 8192 pairs (the largest one-launch call) with scores
    from five integers (runs of ties); 1024 experts (host quotas copied, not
    passed by value) with quotas of 0, all and more than all; quotas on the
    device; expert ids out of range and tokens out of order (flagged, pos -1)."""
    rng = np.random.default_rng(21)
    flags = 0
    if case == "tiny_fp32":
        spec = synth.CONFIGS[1]
        r = synth.make_routing(spec["T"], spec["E"], spec["k"], spec["zipf"], "cfg", 1)
        s = (rng.standard_normal(r.N) ** 2).astype(np.float32)
        q = np.asarray(synth._quotas(1, r, None)["quota"], np.int64)
    else:
        N, E = {"ties_8192": (8192, 64), "wide_1024": (2048, 1024),
                "device_quota": (4096, 256), "bad_indices": (4096, 16)}[case]
        expert = np.minimum(rng.zipf(1.3, N) - 1, E - 1).astype(np.int32)
        token = np.sort(rng.integers(0, N // 4, N)).astype(np.int32)
        if case == "bad_indices":
            expert[rng.integers(0, N, 40)] = E
            expert[rng.integers(0, N, 40)] = -1
            token[100], token[101] = token[101] + 1, token[100]
        r = synth.Routing(N // 4, E, 1, expert, token, rng.random(N).astype(np.float32),
                          np.bincount(expert[(expert >= 0) & (expert < E)], minlength=E), {})
        if case == "ties_8192":
            s = rng.integers(0, 5, N).astype(np.float32)
        else:
            s = (rng.standard_normal(N) ** 2).astype(np.float32)
        c = r.counts
        q = (c // 3 + (np.arange(E) % 3)).astype(np.int64)
        if case == "wide_1024":
            q[::7] = 0
            q[1::7] = c[1::7]
            q[2::7] = c[2::7] + 9
    quota = q
    if case == "device_quota":
        flags = L.LRM_QUOTA_ON_DEVICE
        quota = torch.as_tensor(q.astype(np.int32), device=DEV)
    res = {}
    for one in ("1", "0"):
        monkeypatch.setenv("LRM_SELECT_ONE_LAUNCH", one)
        say("select one launch", case, one, r.N, r.E)
        pos, offsets, kept, ws = _select(L, r, s, quota, flags)
        err = int(ws[:4].cpu().numpy().view(np.uint32)[0])
        res[one] = (pos, offsets, kept[: max(int(offsets[-1]), 0)], err)
    for a, b, name in zip(res["1"], res["0"], ("pos", "offsets", "kept", "err")):
        assert np.array_equal(np.asarray(a), np.asarray(b)), name
    assert (res["1"][3] != 0) == (case == "bad_indices")


@pytest.mark.parametrize("ties", [False, True])
def test_select_run_boundaries(L, ties):
    """Experts at the per-expert selection's size boundaries: 8192 candidates
    (the last size held in registers, 8 per thread), 8193 (keys read from
    memory, a second round of one candidate), 16385 and 1; quotas of one
    candidate, half, and all but one.  With ties: a handful of integer scores,
    zeros among them, so the threshold falls in runs of equal keys that cross
    thread and round boundaries."""
    say("select boundaries", ties)
    sizes = [8192, 8193, 16385, 1, 3]
    E = len(sizes) * 3
    rng = np.random.default_rng(11 + ties)
    expert = np.concatenate([np.full(n, e, np.int32)
                             for e, n in enumerate(sizes * 3)])
    order = rng.permutation(expert.size)
    expert = expert[order]
    N = expert.size
    r = synth.Routing(N, E, 1, expert, np.arange(N, dtype=np.int32),
                      rng.random(N).astype(np.float32), np.bincount(expert, minlength=E), {})
    if ties:
        s = rng.integers(0, 5, N).astype(np.float32)
    else:
        s = (rng.standard_normal(N) ** 2 * 1e-3).astype(np.float32)
    c = r.counts
    q = np.concatenate([np.ones(len(sizes)), c[len(sizes):2 * len(sizes)] // 2,
                        np.maximum(c[2 * len(sizes):] - 1, 0)]).astype(np.int64)
    pos, offsets, kept, _ = _select(L, r, s, q)
    ora = O.select_top_quota(r.expert, s.astype(np.float64), q, E)
    gk = kept_from_pos(pos, r.expert, E)
    for e in range(E):
        assert np.array_equal(gk[e], ora[e]), f"expert {e} ({c[e]} candidates, quota {q[e]})"
    check_packing(pos, offsets, r.expert, E)
    M = offsets[-1]
    assert np.array_equal(kept[:M], np.concatenate(ora))


def test_select_keep_all_and_index_errors(L):
    say("select keep_all / index errors")
    p = synth.make_linear(128, 5, 2, 16, 16, dtype="f32", seed=6)
    r = p["routing"]
    pos, offsets, kept, ws = _select(L, r, np.zeros(r.N), None, flags=L.LRM_KEEP_ALL)
    assert np.all(pos >= 0)
    check_packing(pos, offsets, r.expert, r.E)
    assert L.lrm_check_device_errors(ws) == L.LRM_OK
    # out-of-range experts are reported and treated as absent
    bad = r.expert.copy()
    bad[[3, 50]] = [r.E + 2, -1]
    r2 = synth.Routing(r.T, r.E, r.k, bad, r.token, r.weight, r.counts, {})
    q = np.full(r.E, 1000, np.int32)
    pos, offsets, kept, ws = _select(L, r2, np.ones(r.N), q)
    assert pos[3] == -1 and pos[50] == -1
    assert offsets[-1] == r.N - 2
    assert L.lrm_check_device_errors(ws) == 8  # LRM_ERR_INDEX
    assert L.lrm_check_device_errors(ws) == L.LRM_OK  # cleared


# ------------------------------------------- compact, GEMM, unpermute alone

def _oracle_packing(p, kept_sets):
    r = p["routing"]
    offsets, kept_list, pos = O.pack(kept_sets, r.N)
    return offsets.astype(np.int32), kept_list.astype(np.int32), pos.astype(np.int32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compact_gemm_unpermute_steps(L, dtype):
    say("steps", dtype)
    d_in, d_out = (72, 40) if dtype == "f32" else (264, 136)  # several tiles + ragged tails
    p = synth.make_linear(900, 7, 3, d_in, d_out, dtype=dtype, seed=7, zipf=1.0,
                          quota=lambda c: (2 * c) // 3)
    r = p["routing"]
    kept_sets = O.select_top_quota(r.expert, O.linear_scores(p), p["quota"], r.E)
    offsets, kept_list, pos = _oracle_packing(p, kept_sets)
    M = int(offsets[-1])
    max_rows = M + 5
    pairs = L.Pairs.from_routing(r, DEV)
    X, G, W = (p[k].to(DEV) for k in ("X", "G", "W"))
    dt = X.dtype
    t_off = torch.as_tensor(offsets, device=DEV)
    t_kept = torch.as_tensor(kept_list, device=DEV)
    Xp = torch.zeros(max_rows, d_in, dtype=dt, device=DEV)
    Gp = torch.zeros(max_rows, d_out, dtype=dt, device=DEV)
    L.lrm_compact(pairs, t_kept, t_off, max_rows, L.mat(X, "token"), L.mat(G, "pair"), Xp, Gp)
    torch.cuda.synchronize()
    # Gp is an exact row copy; Xp = w * x rounded once to the input dtype
    g_ref = O.pair_rows(p["G"], "pair", r.token, kept_list)
    assert np.array_equal(Gp[:M].float().cpu().numpy().astype(np.float64), g_ref)
    x_ref = r.weight[kept_list].astype(np.float64)[:, None] * O.pair_rows(p["X"], "token",
                                                                          r.token, kept_list)
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    np.testing.assert_allclose(Xp[:M].float().cpu().numpy(), x_ref, rtol=ulp, atol=1e-30)
    dW = torch.full((r.E, d_out, d_in), float("nan"), device=DEV)
    dXp = torch.full((max_rows, d_in), float("nan"), device=DEV)
    L.lrm_grouped_bwd(r.E, t_off, max_rows, Gp, Xp, W, d_in, d_out, dW, dXp)
    torch.cuda.synchronize()
    # reference products on the GPU's own packed operands (exact fp64 sums)
    Gp64 = Gp[:M].double().cpu().numpy()
    Xp64 = Xp[:M].double().cpu().numpy()
    tol = TOL[dtype] / 20
    for e in range(r.E):
        a, b = offsets[e], offsets[e + 1]
        ref = Gp64[a:b].T @ Xp64[a:b]
        got = dW[e].cpu().numpy()
        if a == b:
            assert not got.any()
        else:
            assert rel_fro(got, ref) < tol, e
        refx = Gp64[a:b] @ O.f64(p["W"][e])
        assert rel_fro(dXp[a:b].cpu().numpy(), refx) < tol, e
    assert torch.isnan(dXp[M:]).all(), "rows past the kept count must stay untouched"
    dX = torch.full((r.T, d_in), float("nan"), device=DEV)
    L.lrm_unpermute(pairs, torch.as_tensor(pos, device=DEV), dXp, d_in, "token", dX)
    torch.cuda.synchronize()
    dxp = dXp[:M].double().cpu().numpy()
    ref = np.zeros((r.T, d_in))
    np.add.at(ref, r.token[kept_list], r.weight[kept_list].astype(np.float64)[:, None] * dxp)
    assert rel_fro(dX.cpu().numpy(), ref) < 1e-6
    assert not dX.cpu().numpy()[~np.isin(np.arange(r.T), r.token[kept_list])].any()
    dXpair = torch.full((r.N, d_in), float("nan"), device=DEV)
    L.lrm_unpermute(pairs, torch.as_tensor(pos, device=DEV), dXp, d_in, "pair", dXpair)
    torch.cuda.synchronize()
    refp = np.zeros((r.N, d_in))
    refp[kept_list] = r.weight[kept_list].astype(np.float64)[:, None] * dxp
    assert rel_fro(dXpair.cpu().numpy(), refp) < 1e-6


def test_gemm_zero_rows_and_heavy_expert(L):
    """M = 0 everywhere (all dW zero), then one expert holding 3000 rows."""
    say("gemm zero/heavy")
    E, d_in, d_out = 6, 128, 256
    W = synth.normal((E, d_out, d_in), 0.02, torch.bfloat16, DEV, "t", 1)
    for sizes in ([0] * E, [0, 3000, 0, 1, 129, 0]):
        offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        M = int(offsets[-1])
        rows = max(M, 1)
        Gp = synth.normal((rows, d_out), 1.0, torch.bfloat16, DEV, "t", 2)
        Xp = synth.normal((rows, d_in), 1.0, torch.bfloat16, DEV, "t", 3)
        dW = torch.full((E, d_out, d_in), float("nan"), device=DEV)
        dXp = torch.full((rows, d_in), float("nan"), device=DEV)
        L.lrm_grouped_bwd(E, torch.as_tensor(offsets, device=DEV), M, Gp, Xp, W, d_in, d_out,
                          dW, dXp)
        torch.cuda.synchronize()
        G64, X64 = Gp.double().cpu().numpy(), Xp.double().cpu().numpy()
        for e in range(E):
            a, b = offsets[e], offsets[e + 1]
            got = dW[e].cpu().numpy()
            if a == b:
                assert not got.any()
            else:
                assert rel_fro(got, G64[a:b].T @ X64[a:b]) < 1e-3
                assert rel_fro(dXp[a:b].cpu().numpy(),
                               G64[a:b] @ O.f64(W[e].cpu())) < 1e-3


@pytest.mark.parametrize("tile", ["S", "M", "L", "X"])
def test_gemm_tile_configs(L, tile, monkeypatch):
    """Every bf16 tile configuration on ragged shapes: empty, 1-row and
    tile-edge experts, a column count and a k extent that leave partial tiles."""
    monkeypatch.setenv("LRM_GEMM_TILE", tile)
    say("gemm tile", tile)
    E, d_in, d_out = 8, 320, 200
    sizes = [0, 1, 63, 64, 65, 257, 700, 0]
    W = synth.normal((E, d_out, d_in), 0.02, torch.bfloat16, DEV, "tc", 1)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offsets[-1])
    Gp = synth.normal((M, d_out), 1.0, torch.bfloat16, DEV, "tc", 2)
    Xp = synth.normal((M, d_in), 1.0, torch.bfloat16, DEV, "tc", 3)
    dW = torch.full((E, d_out, d_in), float("nan"), device=DEV)
    dXp = torch.full((M, d_in), float("nan"), device=DEV)
    L.lrm_grouped_bwd(E, torch.as_tensor(offsets, device=DEV), M, Gp, Xp, W, d_in, d_out, dW,
                      dXp)
    torch.cuda.synchronize()
    G64, X64 = Gp.double().cpu().numpy(), Xp.double().cpu().numpy()
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        got = dW[e].cpu().numpy()
        if a == b:
            assert not got.any()
            continue
        assert rel_fro(got, G64[a:b].T @ X64[a:b]) < 1e-5
        assert rel_fro(dXp[a:b].cpu().numpy(), G64[a:b] @ O.f64(W[e].cpu())) < 1e-5


@pytest.mark.parametrize("d_out", [320, 200])
def test_gemm_lds_dma_bit_exact(L, d_out, monkeypatch):
    """The 256x256 kernels that load operand tiles straight into LDS and read
    the k-strided ones with transposing LDS reads (LRM_GEMM_DMA=2: k-tiles of
    64, two stages; 4: k-tiles of 32, four stages) give the register path's
    results bit for bit (the same MFMAs in the same order on the same
    operands), on empty, 1-row and tile-edge experts and a partial last column
    tile.  With d_out = 200, dX's K is not a whole number of k-tiles and dX
    stays on the register path."""
    monkeypatch.setenv("LRM_GEMM_TILE", "L")
    E, d_in = 8, 200
    sizes = [0, 1, 63, 64, 65, 257, 700, 0]
    W = synth.normal((E, d_out, d_in), 0.02, torch.bfloat16, DEV, "dma", 1)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offsets[-1])
    Gp = synth.normal((M, d_out), 1.0, torch.bfloat16, DEV, "dma", 2)
    Xp = synth.normal((M, d_in), 1.0, torch.bfloat16, DEV, "dma", 3)
    off = torch.as_tensor(offsets, device=DEV)
    res = {}
    for dma in ("0", "2", "4"):
        say("gemm lds dma", d_out, dma)
        monkeypatch.setenv("LRM_GEMM_DMA", dma)
        dW = torch.full((E, d_out, d_in), float("nan"), device=DEV)
        dXp = torch.full((M, d_in), float("nan"), device=DEV)
        L.lrm_grouped_bwd(E, off, M, Gp, Xp, W, d_in, d_out, dW, dXp)
        torch.cuda.synchronize()
        res[dma] = (dW.cpu(), dXp.cpu())
    for dma in ("2", "4"):
        assert torch.equal(res[dma][0], res["0"][0]), f"dW, LRM_GEMM_DMA={dma}"
        assert torch.equal(res[dma][1], res["0"][1]), f"dX, LRM_GEMM_DMA={dma}"
    dW, dXp = res["2"]
    G64, X64 = Gp.double().cpu().numpy(), Xp.double().cpu().numpy()
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            assert not dW[e].numpy().any()
            continue
        assert rel_fro(dW[e].numpy(), G64[a:b].T @ X64[a:b]) < 1e-5
        assert rel_fro(dXp[a:b].numpy(), G64[a:b] @ O.f64(W[e].cpu())) < 1e-5


@pytest.mark.parametrize("tile", ["L", "X"])
@pytest.mark.parametrize("d_out", [512, 768])
def test_dw_heavy_expert_stripes(L, d_out, tile, monkeypatch):
    """dW tiles of heavy experts (one tile at least a quarter of a CU's ideal
    load) are dealt to the 8 XCDs in stripes, the other experts' tiles in
    equal-cost contiguous shares.  Four heavy experts among 100, 8 tiles per
    expert (d_out 512: one tile per stripe) or 12 (d_out 768: stripes of 1 and
    2 tiles), one block per tile (L) and persistent blocks (X): every expert's
    dW against the fp64 product, outputs prefilled with NaN so that a tile
    left out shows."""
    monkeypatch.setenv("LRM_GEMM_TILE", tile)
    d_in = 1024
    rng = np.random.default_rng(11)
    sizes = rng.integers(20, 41, 100)
    sizes[[7, 50]] = 2500
    sizes[[20, 81]] = 300
    sizes[33] = 0
    E = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offsets[-1])
    say("dw heavy stripes", d_out, tile, M)
    W = synth.normal((E, d_out, d_in), 0.02, torch.bfloat16, DEV, "stripe", 1)
    Gp = synth.normal((M, d_out), 1.0, torch.bfloat16, DEV, "stripe", 2)
    Xp = synth.normal((M, d_in), 1.0, torch.bfloat16, DEV, "stripe", 3)
    off = torch.as_tensor(offsets, device=DEV)
    dW = torch.full((E, d_out, d_in), float("nan"), device=DEV)
    L.lrm_grouped_bwd(E, off, M, Gp, Xp, W, d_in, d_out, dW, None)
    torch.cuda.synchronize()
    dW = dW.cpu().numpy()
    G64, X64 = Gp.double().cpu().numpy(), Xp.double().cpu().numpy()
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            assert not dW[e].any(), e
            continue
        assert rel_fro(dW[e], G64[a:b].T @ X64[a:b]) < 1e-5, e


# ------------------------------------------------------------ fused call

@pytest.mark.parametrize("x_rows,g_rows", [("token", "pair"), ("pair", "token")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_linear_small(L, dtype, x_rows, g_rows):
    say("fused linear", dtype, x_rows, g_rows)
    p = synth.make_linear(600, 10, 4, 136, 200, dtype=dtype, x_rows=x_rows, g_rows=g_rows,
                          seed=8, zipf=1.4, quota=lambda c: (c * 5) // 8 + (c % 3 == 0))
    res = run_linear(L, p, DEV)
    s = judge_linear(p, res)
    say("  ", s)


@pytest.mark.parametrize("shape", [(600, 10, 4, 136, 200), (4096, 8, 2, 520, 264)])
def test_fused_linear_dw_bf16_is_rounded_fp32(L, shape):
    """LRM_DW_BF16: dW equals the fp32 path's dW rounded to nearest even, bit
    for bit, and every other output is unchanged (small experts use the 64-row
    dX tiles, large ones the 256x256 tiles; ragged d_in and d_out)."""
    T, E, k, d_in, d_out = shape
    say("fused linear, bf16 dW", shape)
    p = synth.make_linear(T, E, k, d_in, d_out, dtype="bf16", seed=12, zipf=1.2,
                          quota=lambda c: (3 * c) // 4)
    ref = run_linear(L, p, DEV)
    got = run_linear(L, p, DEV, flags=L.LRM_DW_BF16)
    assert got["dW"].dtype == torch.bfloat16
    assert torch.equal(got["dW"].view(torch.int16), ref["dW"].to(torch.bfloat16).view(torch.int16))
    for key in ("dX", "score", "pos", "offsets"):
        assert torch.equal(got[key], ref[key]), key


def test_fused_linear_dw_bf16_needs_bf16_inputs(L):
    import ctypes as C
    p = synth.make_linear(64, 4, 2, 32, 32, dtype="f32", seed=3)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    X, G, W = (p[k].to(DEV) for k in ("X", "G", "W"))
    pb = L.linear_problem(pairs, X, "token", G, "pair", W, p["quota"], L.LRM_DW_BF16)
    out = dict(dW=torch.empty(r.E, 32, 32, device=DEV), dX=torch.empty(r.T, 32, device=DEV))
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    assert L._lib.lrm_workspace_size(C.byref(pb.c)) == 0
    st = L._lib.lrm_expert_backward(C.byref(pb.c), C.byref(L._outputs(out)), ws.data_ptr(),
                                    ws.numel(), None)
    assert st == 10  # LRM_ERR_UNSUPPORTED, before any launch


def test_fused_linear_config1(L):
    p = synth.make_config(1)
    res = run_linear(L, p, DEV)
    s = judge_linear(p, res)
    say("config1", s)
    assert s["kept"] == 253


def test_fused_linear_keep_all_is_unpruned(L):
    p = synth.make_linear(500, 8, 2, 64, 128, dtype="bf16", seed=9, zipf=1.0)
    res = run_linear(L, p, DEV, flags=L.LRM_KEEP_ALL)
    s = judge_linear(p, res, keep_all=True)
    assert s["kept"] == p["routing"].N


def test_fused_linear_quota_zero(L):
    p = synth.make_linear(300, 6, 2, 64, 64, dtype="bf16", seed=10, quota=lambda c: 0 * c)
    res = run_linear(L, p, DEV)
    assert not res["dW"].any() and not res["dX"].any()
    assert (res["pos"].numpy()[: p["routing"].N] == -1).all()


def test_fused_linear_deterministic(L):
    p = synth.make_linear(800, 12, 4, 256, 128, dtype="bf16", seed=11, zipf=1.2)
    a = run_linear(L, p, DEV)
    b = run_linear(L, p, DEV)
    for k in ("dW", "dX", "score", "pos", "offsets"):
        assert torch.equal(a[k], b[k]), k


def test_fused_linear_config2(L):
    """Qwen3-30B-A3B-shaped projection at full size (the benchmark workload)."""
    say("config2: generating")
    p = synth.make_config(2, device=DEV)
    say("config2: running")
    res = run_linear(L, p, DEV)
    say("config2: oracle")
    host = dict(p, X=p["X"].cpu(), G=p["G"].cpu(), W=p["W"].cpu())
    s = judge_linear(host, res)
    say("config2", s)
    assert s["kept"] == int(np.minimum(p["quota"], p["routing"].counts).sum())


def _no_pairs_linear(dtype, T=96, E=5, d_in=64, d_out=48):
    r = synth.Routing(T, E, 2, np.zeros(0, np.int32), np.zeros(0, np.int32),
                      np.zeros(0, np.float32), np.zeros(E, np.int64))
    dt = synth.torch_dtype(dtype)
    g = torch.Generator().manual_seed(11)
    return dict(kind="linear", dtype=dtype, routing=r, T=T, N=0, E=E, k=2, d_in=d_in,
                d_out=d_out, X_rows="token", G_rows="token", quota=np.full(E, 3, np.int32),
                X=torch.randn(T, d_in, generator=g).to(dt),
                G=torch.randn(T, d_out, generator=g).to(dt),
                W=torch.randn(E, d_out, d_in, generator=g).to(dt))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_linear_no_pairs(L, dtype):
    # a GPU whose experts received no pair in this layer call: every output
    # is written, and is exactly zero
    say("fused linear, no pairs", dtype)
    p = _no_pairs_linear(dtype)
    res = run_linear(L, p, DEV)
    assert not torch.any(res["dW"] != 0), "dW must be exactly zero"
    assert not torch.any(res["dX"] != 0), "dX must be exactly zero"
    assert torch.equal(res["offsets"], torch.zeros(p["E"] + 1, dtype=torch.int32))


def test_fused_linear_max_experts(L):
    # the largest expert count the ABI takes: most of the 4096 experts get no
    # pair or one pair, a few get several (Zipf skew)
    say("fused linear, 4096 experts")
    p = synth.make_linear(2048, 4096, 2, 64, 32, dtype="bf16", seed=21, zipf=1.0,
                          quota=lambda c: (2 * c + 1) // 3)
    s = judge_linear(p, run_linear(L, p, DEV))
    say("  ", s)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_linear_quota_on_device(L, dtype):
    # the same quotas read from device memory (LRM_QUOTA_ON_DEVICE): the same
    # kept sets and bit-identical gradients (the packed blocks are sized for
    # every pair, which may pick other tile shapes; each output element is the
    # same sum in the same order)
    say("fused linear, device quotas", dtype)
    p = synth.make_linear(600, 10, 4, 136, 200, dtype=dtype, seed=8, zipf=1.4,
                          quota=lambda c: (c * 5) // 8 + (c % 3 == 0))
    host = run_linear(L, p, DEV)
    pd = dict(p, quota=torch.tensor(p["quota"], dtype=torch.int32, device=DEV))
    dev = run_linear(L, pd, DEV, flags=L.LRM_QUOTA_ON_DEVICE)
    for k in ("pos", "offsets", "dW", "dX", "score"):
        assert torch.equal(torch.nan_to_num(host[k].float()), torch.nan_to_num(dev[k].float())), k
    judge_linear(p, dev)


def test_fused_linear_debug_checks(L):
    # an expert id out of range: without LRM_DEBUG_CHECKS the call succeeds and
    # lrm_check_device_errors reports it; with the flag the call itself does
    say("fused linear, debug checks")
    p = synth.make_linear(64, 4, 2, 32, 32, dtype="bf16", seed=9)
    r = p["routing"]
    r.expert = r.expert.copy()
    r.expert[5] = r.E + 3
    res = run_linear(L, p, DEV)
    assert L.lrm_check_device_errors(res["ws"]) == L.LRM_ERR_INDEX
    with pytest.raises(L.LrmError) as ex:
        run_linear(L, p, DEV, flags=L.LRM_DEBUG_CHECKS)
    assert ex.value.status == L.LRM_ERR_INDEX
    # a clean call after it reports no error
    p2 = synth.make_linear(64, 4, 2, 32, 32, dtype="bf16", seed=9)
    res = run_linear(L, p2, DEV, flags=L.LRM_DEBUG_CHECKS)
    judge_linear(p2, res)


def _graph_replays(L, pb, out, ws, n=3):
    """Capture one fused call in a HIP graph, replay it n times with eager work
    in between (the outputs overwritten), and return the outputs of each replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.lrm_expert_backward(pb, out, ws=ws)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.lrm_expert_backward(pb, out, ws=ws)
    got = []
    for _ in range(n):
        for v in out.values():  # eager work between the replays
            v.fill_(-7) if v.dtype == torch.int32 else v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got.append({k: v.cpu().clone() for k, v in out.items()})
    return got


def test_fused_linear_graph_replay(L):
    # the fused call is only kernel launches (host quotas go in the kernel
    # arguments), so it can be captured in a HIP graph and replayed
    say("fused linear, graph replay")
    p = synth.make_linear(600, 10, 4, 136, 200, dtype="bf16", seed=8, zipf=1.4,
                          quota=lambda c: (c * 5) // 8 + (c % 3 == 0))
    eager = run_linear(L, p, DEV)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    X, G, W = (p[k].to(DEV) for k in ("X", "G", "W"))
    pb = L.linear_problem(pairs, X, "token", G, "pair", W, p["quota"])
    out = dict(dW=torch.empty(r.E, p["d_out"], p["d_in"], device=DEV),
               dX=torch.empty(r.T, p["d_in"], device=DEV),
               pos=torch.empty(r.N, dtype=torch.int32, device=DEV),
               offsets=torch.empty(r.E + 1, dtype=torch.int32, device=DEV))
    ws = torch.empty(L.lrm_workspace_size(pb), dtype=torch.uint8, device=DEV)
    for got in _graph_replays(L, pb, out, ws):
        for k in out:
            assert torch.equal(got[k], eager[k]), k


def test_capture_refused_for_copied_host_quotas(L):
    """Host quotas of more than 512 experts travel by a stream copy of the
    host array, which a replay would repeat while the packed sizes stay those
    of the capture: on a capturing stream the call is refused before any
    launch (LRM_ERR_UNSUPPORTED = 10).  Device quotas of the same problem
    capture and replay bit-exactly against the eager call."""
    say("capture with 600 experts' host quotas")
    p = synth.make_linear(900, 600, 2, 64, 64, dtype="bf16", seed=31, zipf=1.1,
                          quota=lambda c: (c + 1) // 2)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    X, G, W = (p[k].to(DEV) for k in ("X", "G", "W"))
    pb = L.linear_problem(pairs, X, "token", G, "pair", W, p["quota"])
    out = dict(dW=torch.empty(r.E, 64, 64, device=DEV), dX=torch.empty(r.T, 64, device=DEV))
    ws = torch.empty(L.lrm_workspace_size(pb), dtype=torch.uint8, device=DEV)
    L.lrm_expert_backward(pb, out, ws=ws)  # eager: fine
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(L.LrmError) as ei:
        with torch.cuda.graph(graph):
            L.lrm_expert_backward(pb, out, ws=ws)
    assert ei.value.status == 10, str(ei.value)
    torch.cuda.synchronize()
    qd = torch.tensor(p["quota"], dtype=torch.int32, device=DEV)
    pbd = L.linear_problem(pairs, X, "token", G, "pair", W, qd, L.LRM_QUOTA_ON_DEVICE)
    outd = dict(dW=torch.empty(r.E, 64, 64, device=DEV), dX=torch.empty(r.T, 64, device=DEV),
                pos=torch.empty(r.N, dtype=torch.int32, device=DEV))
    wsd = torch.empty(L.lrm_workspace_size(pbd), dtype=torch.uint8, device=DEV)
    L.lrm_expert_backward(pbd, outd, ws=wsd)
    torch.cuda.synchronize()
    eager = {k: v.cpu().clone() for k, v in outd.items()}
    for got in _graph_replays(L, pbd, outd, wsd):
        for k in outd:
            assert torch.equal(got[k], eager[k]), k


@pytest.mark.parametrize("x_rows,g_rows", [("token", "pair"), ("pair", "token")])
@pytest.mark.parametrize("tile", ["L", "X"])
def test_fused_linear_gather_loads_bit_exact(L, x_rows, g_rows, tile, monkeypatch):
    """LRM_GATHER_LOADS: the dW GEMM gathers w x from X in its loader instead
    of reading the packed copy; every output must equal the call without the
    flag bit for bit (ragged shapes, experts that keep 0..all rows), with
    fp32 and bf16 weight gradients."""
    monkeypatch.setenv("LRM_GEMM_TILE", tile)
    say("gather loads, linear", x_rows, g_rows, tile)
    p = synth.make_linear(700, 10, 4, 200, 136, dtype="bf16", x_rows=x_rows, g_rows=g_rows,
                          seed=19, zipf=1.4, quota=lambda c: (c * 5) // 8 + (c % 3 == 0))
    for extra in (0, L.LRM_DW_BF16):
        ref = run_linear(L, p, DEV, flags=extra)
        got = run_linear(L, p, DEV, flags=extra | L.LRM_GATHER_LOADS)
        for k in ("dW", "dX", "score", "pos", "offsets"):
            assert torch.equal(got[k].view(torch.int16) if got[k].dtype == torch.bfloat16
                               else got[k], ref[k].view(torch.int16)
                               if ref[k].dtype == torch.bfloat16 else ref[k]), (k, extra)
    judge_linear(p, got)


def test_fused_linear_config2_gather_loads(L):
    p = synth.make_config(2, device=DEV)
    ref = run_linear(L, p, DEV)
    got = run_linear(L, p, DEV, flags=L.LRM_GATHER_LOADS)
    for k in ("dW", "dX", "pos", "offsets"):
        assert torch.equal(got[k], ref[k]), k
