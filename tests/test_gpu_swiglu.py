"""GPU parity of the SwiGLU expert backward (down -> gate/up, each projection
with its own LRM scores and quotas) through the fused C-ABI call, against the
fp64 oracle."""

import numpy as np
import pytest
import torch

from pruned_expert_backward_lrm_amd import synth

from parity import judge_swiglu, run_swiglu

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


QUOTAS = {
    # gate/up quotas at least the down quotas: the second selection keeps all
    "same": (lambda c: c // 2, lambda c: c // 2, lambda c: c // 2),
    # a real second selection with different gate and up quotas
    "second": (lambda c: (3 * c) // 4, lambda c: (3 * c) // 8 + 1, lambda c: c // 3),
}


@pytest.mark.parametrize("variant", ["same", "second"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_swiglu_small(L, dtype, variant):
    say("swiglu small", dtype, variant)
    p = synth.make_swiglu(400, 6, 2, 136, 72, dtype=dtype, seed=5, zipf=1.2,
                          quotas=QUOTAS[variant], g_std=1e-2)
    s = judge_swiglu(p, run_swiglu(L, p, DEV))
    say("  ", s)


@pytest.mark.parametrize("tile", ["S", "M", "L", "X"])
@pytest.mark.parametrize("variant", ["same", "second"])
def test_fused_swiglu_tile_configs(L, variant, tile, monkeypatch):
    """Every bf16 GEMM tile configuration inside the fused SwiGLU call: the
    dual-K input-gradient product (same quotas) and the separate gate/up
    products (second selection); H and I leave partial tiles."""
    monkeypatch.setenv("LRM_GEMM_TILE", tile)
    say("swiglu tiles", variant, tile)
    p = synth.make_swiglu(700, 6, 2, 200, 136, dtype="bf16", seed=15, zipf=1.2,
                          quotas=QUOTAS[variant], g_std=1e-2)
    s = judge_swiglu(p, run_swiglu(L, p, DEV))
    say("  ", s)


def test_fused_swiglu_keep_all(L):
    p = synth.make_swiglu(300, 5, 2, 128, 64, dtype="bf16", seed=6, zipf=1.0)
    s = judge_swiglu(p, run_swiglu(L, p, DEV, flags=L.LRM_KEEP_ALL), keep_all=True)
    assert s["kept_down"] == p["routing"].N


def test_fused_swiglu_quota_zero(L):
    p = synth.make_swiglu(200, 4, 2, 64, 64, dtype="bf16", seed=7,
                          quotas=(lambda c: 0 * c, lambda c: c, lambda c: c))
    res = run_swiglu(L, p, DEV)
    for k in ("dW_gate", "dW_up", "dW_down", "dX"):
        assert not res[k].any(), k


@pytest.mark.parametrize("variant", ["same", "second"])
def test_fused_swiglu_dw_bf16_is_rounded_fp32(L, variant):
    """LRM_DW_BF16: every weight gradient equals the fp32 path's rounded to
    nearest even, bit for bit; the other outputs are unchanged."""
    say("swiglu bf16 dW", variant)
    p = synth.make_swiglu(700, 6, 2, 200, 136, dtype="bf16", seed=16, zipf=1.2,
                          quotas=QUOTAS[variant], g_std=1e-2)
    ref = run_swiglu(L, p, DEV)
    got = run_swiglu(L, p, DEV, flags=L.LRM_DW_BF16)
    for k in ("dW_gate", "dW_up", "dW_down"):
        assert got[k].dtype == torch.bfloat16
        assert torch.equal(got[k].view(torch.int16), ref[k].to(torch.bfloat16).view(torch.int16)), k
    for k in ("dX", "score", "pos", "score_gate", "pos_gate", "pos_up", "dH"):
        assert torch.equal(got[k], ref[k]), k


@pytest.mark.parametrize("variant", ["same", "second"])
def test_fused_swiglu_h_sumsq_table(L, variant):
    """The down score from a per-pair |silu(a) b|^2 saved by the forward (here
    computed in fp64 on the host): the down scores are w^2 |g|^2 times the
    table, rounded once to fp32, and the whole call meets the parity bar."""
    say("swiglu with a saved |h|^2 table", variant)
    p = synth.make_swiglu(700, 6, 2, 200, 136, dtype="bf16", seed=17, zipf=1.2,
                          quotas=QUOTAS[variant], g_std=1e-2)
    a, b = p["A"].double(), p["B"].double()
    h = a * torch.sigmoid(a) * b
    tab = (h * h).sum(dim=1)
    res = run_swiglu(L, p, DEV, h_sumsq=tab)
    r = p["routing"]
    g2 = (p["G"].double() ** 2).sum(dim=1)
    w = torch.as_tensor(r.weight, dtype=torch.float64)
    tok = torch.as_tensor(r.token, dtype=torch.int64)
    expect = (w * w * g2[tok] * tab).float()
    got = res["score"][: r.N]
    assert torch.allclose(got, expect, rtol=1e-6, atol=0), (got - expect).abs().max()
    s = judge_swiglu(p, res)
    say("  ", s)


@pytest.mark.parametrize("variant", ["same", "second"])
@pytest.mark.parametrize("tile", ["L", "X"])
def test_fused_swiglu_gather_loads_bit_exact(L, variant, tile, monkeypatch):
    """LRM_GATHER_LOADS: the gate and up dW GEMMs gather w x from X in their
    loaders (one shared row map, or one per projection after a second
    selection); every output equals the call without the flag bit for bit."""
    monkeypatch.setenv("LRM_GEMM_TILE", tile)
    say("gather loads, swiglu", variant, tile)
    p = synth.make_swiglu(700, 6, 2, 200, 136, dtype="bf16", seed=18, zipf=1.2,
                          quotas=QUOTAS[variant], g_std=1e-2)
    ref = run_swiglu(L, p, DEV)
    got = run_swiglu(L, p, DEV, flags=L.LRM_GATHER_LOADS)
    for k in ("dW_gate", "dW_up", "dW_down", "dX", "score", "pos", "score_gate", "pos_gate",
              "pos_up", "dH"):
        assert torch.equal(got[k], ref[k]), k
    judge_swiglu(p, got)


@pytest.mark.parametrize("flags", [0, 2])
def test_fused_swiglu_lds_dma_bit_exact(L, flags, monkeypatch):
    """The LDS-DMA 256x256 kernels (LRM_GEMM_DMA=2 and 4) in the fused SwiGLU
    call, fp32 and bf16 (LRM_DW_BF16 = 2) weight gradients, the gate/up dX
    product over its two K segments: every output equals the register path's
    (LRM_GEMM_DMA=0) bit for bit.  H = 320 and I = 192 leave partial column
    tiles and let every product take the DMA kernels."""
    monkeypatch.setenv("LRM_GEMM_TILE", "L")
    p = synth.make_swiglu(900, 6, 2, 320, 192, dtype="bf16", seed=21, zipf=1.2,
                          quotas=QUOTAS["second"], g_std=1e-2)
    res = {}
    for dma in ("0", "2", "4"):
        say("swiglu lds dma", flags, dma)
        monkeypatch.setenv("LRM_GEMM_DMA", dma)
        res[dma] = run_swiglu(L, p, DEV, flags=flags)
    for dma in ("2", "4"):
        for k in ("dW_gate", "dW_up", "dW_down", "dX", "dH"):
            assert torch.equal(res[dma][k], res["0"][k]), (k, dma)
    if flags == 0:
        judge_swiglu(p, res["2"])


@pytest.mark.parametrize("tile", ["S", "M", "L", "X"])
@pytest.mark.parametrize("shape", [(200, 64), (200, 192), (776, 320)])
@pytest.mark.parametrize("flags", [0, 2])
def test_fused_gate_up_dw_bit_exact(L, tile, shape, flags, monkeypatch):
    """Same quotas, bf16, I a multiple of 64: one launch computes dW_gate and
    dW_up over [GA | GB] (2I rows per expert split at I, tiles straddling the
    split), and the dX launch reads GA and GB as two K segments of the
    2I-wide rows.  Every output equals the two-launch path's
    (LRM_FUSE_GATE_UP=0) bit for bit, fp32 and bf16 (LRM_DW_BF16 = 2) weight
    gradients; at H = 776, I = 320 the 256x256 tiles number 12 per expert,
    so the heavy experts' tiles go out in XCD stripes.  Judged against the
    oracle with fp32 weight gradients."""
    H, I = shape
    monkeypatch.setenv("LRM_GEMM_TILE", tile)
    say("fused gate/up dW", tile, shape, flags)
    p = synth.make_swiglu(1200, 8, 2, H, I, dtype="bf16", seed=31, zipf=1.3,
                          quotas=QUOTAS["same"], g_std=1e-2)
    got = run_swiglu(L, p, DEV, flags=flags)
    monkeypatch.setenv("LRM_FUSE_GATE_UP", "0")
    ref = run_swiglu(L, p, DEV, flags=flags)
    for k in ("dW_gate", "dW_up", "dW_down", "dX", "dH", "score", "pos", "score_gate",
              "pos_gate", "pos_up"):
        assert torch.equal(got[k], ref[k]), k
    if flags == 0:
        judge_swiglu(p, got)


def test_fused_swiglu_deterministic(L):
    p = synth.make_swiglu(500, 8, 2, 256, 128, dtype="bf16", seed=8, zipf=1.1,
                          quotas=QUOTAS["second"])
    a = run_swiglu(L, p, DEV)
    b = run_swiglu(L, p, DEV)
    for k in ("dW_gate", "dW_up", "dW_down", "dX", "score", "pos", "score_gate", "pos_gate",
              "pos_up"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("cfg", ["3", "3b", "4", "5"])
def test_swiglu_configs(L, cfg):
    """Full-size SwiGLU workloads, in the launch configuration the benchmark
    times.  Every kept set of the down stage; on configs 3, 3b and 4 the
    gate/up kept sets and weight gradients of every expert and dX of every
    token; on config 5 every expert that kept at most 256 rows (the light
    experts on the small-tile paths) plus the 8 heaviest, and dX of 1024
    sampled tokens.  Gradients are judged expert by expert and per block of
    64 dX rows."""
    import time
    cid = int(cfg[0])
    say(f"config {cfg}: generating")
    p = synth.make_config(cid, device=DEV, variant="3b" if cfg == "3b" else None)
    say(f"config {cfg}: running")
    res = run_swiglu(L, p, DEV)
    host = dict(p, **{k: p[k].cpu() for k in ("X", "G", "A", "B", "W_gate", "W_up", "W_down")})
    r = p["routing"]
    kept = np.diff(res["offsets"].numpy().astype(np.int64))
    t0 = time.perf_counter()
    if cid in (3, 4):
        say(f"config {cfg}: oracle on all {r.E} experts and all {r.T} tokens")
        s = judge_swiglu(host, res)
    else:
        heavy = np.argsort(-kept, kind="stable")[:8]
        ex = sorted(set(np.nonzero(kept <= 256)[0].tolist()) | set(heavy.tolist()))
        rng = np.random.default_rng(cid)
        toks = np.sort(rng.choice(r.T, size=1024, replace=False))
        say(f"config {cfg}: oracle on {len(ex)} experts ({int(kept[ex].sum())} of "
            f"{int(kept.sum())} kept rows), dX of {toks.size} tokens")
        s = judge_swiglu(host, res, experts=ex, tokens=toks)
    say(f"config {cfg} ({time.perf_counter() - t0:.1f} s of oracle)", s)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_swiglu_no_pairs(L, dtype):
    # no pair on this GPU: every weight gradient and every dX row is exactly 0
    say("swiglu, no pairs", dtype)
    T, E, H, I = 80, 4, 64, 32
    r = synth.Routing(T, E, 2, np.zeros(0, np.int32), np.zeros(0, np.int32),
                      np.zeros(0, np.float32), np.zeros(E, np.int64))
    dt = synth.torch_dtype(dtype)
    g = torch.Generator().manual_seed(12)
    q = np.full(E, 2, np.int32)
    p = dict(kind="swiglu", dtype=dtype, routing=r, T=T, N=0, E=E, k=2, H=H, I=I,
             quota_down=q, quota_gate=q.copy(), quota_up=q.copy(),
             X=torch.randn(T, H, generator=g).to(dt), G=torch.randn(T, H, generator=g).to(dt),
             A=torch.zeros(0, I).to(dt), B=torch.zeros(0, I).to(dt),
             W_gate=torch.randn(E, I, H, generator=g).to(dt),
             W_up=torch.randn(E, I, H, generator=g).to(dt),
             W_down=torch.randn(E, H, I, generator=g).to(dt))
    res = run_swiglu(L, p, DEV)
    for k in ("dW_gate", "dW_up", "dW_down", "dX"):
        assert not torch.any(res[k] != 0), f"{k} must be exactly zero"
    assert torch.equal(res["offsets"], torch.zeros(E + 1, dtype=torch.int32))


@pytest.mark.parametrize("variant", ["same", "second"])
def test_fused_swiglu_quota_on_device(L, variant):
    # quotas in device memory: the call always runs the gate/up selections
    # (the host cannot compare the quotas), so the result must meet the oracle;
    # with a real second selection both runs take that path and agree bit for bit
    say("swiglu, device quotas", variant)
    p = synth.make_swiglu(400, 6, 2, 136, 72, dtype="bf16", seed=5, zipf=1.2,
                          quotas=QUOTAS[variant], g_std=1e-2)
    t = lambda q: torch.tensor(q, dtype=torch.int32, device=DEV)  # noqa: E731
    pd = dict(p, quota_down=t(p["quota_down"]), quota_gate=t(p["quota_gate"]),
              quota_up=t(p["quota_up"]))
    dev = run_swiglu(L, pd, DEV, flags=L.LRM_QUOTA_ON_DEVICE)
    judge_swiglu(p, dev)
    if variant == "second":
        host = run_swiglu(L, p, DEV)
        for k in ("dW_gate", "dW_up", "dW_down", "dX", "pos", "offsets"):
            assert torch.equal(torch.nan_to_num(host[k].float()), torch.nan_to_num(dev[k].float())), k


@pytest.mark.parametrize("variant", ["same", "second"])
def test_fused_swiglu_graph_replay(L, variant):
    say("swiglu, graph replay", variant)
    from test_gpu_linear import _graph_replays
    p = synth.make_swiglu(400, 6, 2, 136, 72, dtype="bf16", seed=5, zipf=1.2,
                          quotas=QUOTAS[variant], g_std=1e-2)
    eager = run_swiglu(L, p, DEV)
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, DEV)
    t = {k: p[k].to(DEV) for k in ("X", "G", "A", "B", "W_gate", "W_up", "W_down")}
    pb = L.swiglu_problem(pairs, t["X"], "token", t["G"], "token", t["A"], t["B"], t["W_gate"],
                          t["W_up"], t["W_down"], p["quota_down"], p["quota_gate"], p["quota_up"])
    E, H, I = r.E, p["H"], p["I"]
    out = dict(dW_gate=torch.empty(E, I, H, device=DEV), dW_up=torch.empty(E, I, H, device=DEV),
               dW_down=torch.empty(E, H, I, device=DEV), dX=torch.empty(r.T, H, device=DEV),
               pos=torch.empty(r.N, dtype=torch.int32, device=DEV))
    ws = torch.empty(L.lrm_workspace_size(pb), dtype=torch.uint8, device=DEV)
    for got in _graph_replays(L, pb, out, ws):
        for k in out:
            assert torch.equal(got[k], eager[k]), k
