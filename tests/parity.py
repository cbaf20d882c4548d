"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and judge it against the fp64 oracle.

Parity rule for selections (several kept sets can be correct when scores tie
or nearly tie): the GPU keeps exactly M_e = min(q_e, n_e) pairs per expert,
and every pair in the symmetric difference with the oracle's kept set has an
oracle score within 1e-6 relative of the expert's threshold tau_e (the
oracle's M_e-th largest score).  Gradients are then compared with the oracle
re-run on the GPU's kept sets, by relative Frobenius error: 1e-5 for fp32
inputs, 2e-2 for bf16 inputs with fp32 accumulation, asserted for every
expert's weight gradient on its own and for every block of 64 dX rows on its
own (a whole-tensor norm would let one wrong light expert hide under the
others); the whole-tensor errors are kept as a summary.  Experts with nothing
kept and rows with no kept pair must be exactly zero.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import lrm_oracle as O

TOL = {"f32": 1e-5, "bf16": 2e-2}
WINDOW = 1e-6


def rel_fro(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    d = np.linalg.norm(got - ref)
    return float(d / n) if n > 0 else float(d)


DX_BLOCK = 64


def check_per_expert(name, got, ref, experts, kept_sizes, tol):
    """Relative Frobenius error of every listed expert's gradient on its own:
    <= tol where the expert kept something, exactly zero where it kept
    nothing.  got[e], ref[e] indexable by expert.  Returns the largest error."""
    worst = 0.0
    for e in experts:
        g = np.asarray(got[e], np.float64)
        if kept_sizes[e] == 0:
            assert not g.any(), f"{name} expert {e} kept nothing but is not 0"
            continue
        err = rel_fro(g, ref[e])
        assert err <= tol, f"{name} expert {e} ({kept_sizes[e]} rows): rel err {err}"
        worst = max(worst, err)
    return worst


def check_row_blocks(name, got, ref, tol, block=DX_BLOCK):
    """Relative Frobenius error of every block of `block` rows on its own, and
    rows whose reference is zero (nothing kept) exactly zero.  Returns the
    largest block error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    zero = ~np.any(ref != 0, axis=1)
    assert not np.any(got[zero]), f"{name}: rows without kept pairs must be 0"
    worst = 0.0
    for r0 in range(0, got.shape[0], block):
        if not np.any(ref[r0:r0 + block]):
            continue
        err = rel_fro(got[r0:r0 + block], ref[r0:r0 + block])
        assert err <= tol, f"{name}: rows {r0}..{r0 + block - 1} rel err {err}"
        worst = max(worst, err)
    return worst


def kept_from_pos(pos: np.ndarray, ids_expert: np.ndarray, E: int) -> list[np.ndarray]:
    """Per-expert kept ids (ascending) from a pos array (-1 = dropped)."""
    pos = np.asarray(pos)
    out = []
    for e in range(E):
        ids = np.nonzero((ids_expert == e) & (pos >= 0))[0]
        out.append(ids)
    return out


def check_packing(pos, offsets, expert_of_id, E):
    """Packed rows are expert blocks back to back with ids ascending inside."""
    pos = np.asarray(pos).astype(np.int64)
    offsets = np.asarray(offsets).astype(np.int64)
    assert offsets[0] == 0 and np.all(np.diff(offsets) >= 0)
    for e in range(E):
        ids = np.nonzero((expert_of_id == e) & (pos >= 0))[0]
        assert ids.shape[0] == offsets[e + 1] - offsets[e], f"expert {e}: block size"
        assert np.array_equal(pos[ids], np.arange(offsets[e], offsets[e + 1])), \
            f"expert {e}: rows not ascending in id"
    assert np.all(pos[(expert_of_id < 0) | (expert_of_id >= E)] == -1)


def check_selection(gpu_kept, ora_kept, score64, counts, label=""):
    """Kept-set parity with the threshold window.  Returns #pairs that differ."""
    ndiff = 0
    for e, (g, o) in enumerate(zip(gpu_kept, ora_kept)):
        assert g.shape[0] == o.shape[0], f"{label} expert {e}: |K| {g.shape[0]} != {o.shape[0]}"
        diff = np.setxor1d(g, o)
        if diff.size == 0:
            continue
        tau = O.threshold(score64, o, int(counts[e]))
        assert tau is not None, f"{label} expert {e}: sets differ with nothing to choose"
        bad = diff[np.abs(score64[diff] - tau) > WINDOW * tau]
        assert bad.size == 0, f"{label} expert {e}: pairs {bad[:8]} differ away from threshold"
        ndiff += diff.size
    return ndiff


def to_dev(t, device):
    return t.to(device) if isinstance(t, torch.Tensor) else t


def run_linear(L, p: dict, device: str, flags: int = 0, ws=None):
    """The fused LINEAR backward through the C ABI.  Returns host tensors."""
    r = p["routing"]
    pairs = L.Pairs.from_routing(r, device)
    X, G, W = (p[k].to(device) for k in ("X", "G", "W"))
    pb = L.linear_problem(pairs, X, p["X_rows"], G, p["G_rows"], W,
                          None if flags & L.LRM_KEEP_ALL else p["quota"], flags)
    rows = r.T if p["X_rows"] == "token" else r.N
    f32, i32 = dict(dtype=torch.float32, device=device), dict(dtype=torch.int32, device=device)
    wdt = torch.bfloat16 if flags & L.LRM_DW_BF16 else torch.float32
    out = dict(dW=torch.full((r.E, p["d_out"], p["d_in"]), float("nan"), dtype=wdt,
                             device=device),
               dX=torch.full((rows, p["d_in"]), float("nan"), **f32),
               score=torch.full((max(r.N, 1),), float("nan"), **f32),
               pos=torch.full((max(r.N, 1),), -7, **i32),
               offsets=torch.full((r.E + 1,), -7, **i32))
    ws = L.lrm_expert_backward(pb, out, ws=ws)
    torch.cuda.synchronize()
    res = {k: v.cpu() for k, v in out.items()}
    res["ws"] = ws
    return res


def run_swiglu(L, p: dict, device: str, flags: int = 0, ws=None, h_sumsq=None):
    """The fused SwiGLU backward through the C ABI, with every optional output
    requested.  Returns host tensors."""
    r = p["routing"]
    keep_all = bool(flags & L.LRM_KEEP_ALL)
    pairs = L.Pairs.from_routing(r, device)
    t = {k: p[k].to(device) for k in ("X", "G", "A", "B", "W_gate", "W_up", "W_down")}
    q = (None, None, None) if keep_all else (p["quota_down"], p["quota_gate"], p["quota_up"])
    hs = None if h_sumsq is None else h_sumsq.to(device=device, dtype=torch.float64)
    pb = L.swiglu_problem(pairs, t["X"], "token", t["G"], "token", t["A"], t["B"], t["W_gate"],
                          t["W_up"], t["W_down"], *q, flags, h_sumsq=hs)
    H, I, E, N = p["H"], p["I"], r.E, r.N
    qd = p["quota_down"]
    qd_host = qd.cpu().numpy() if isinstance(qd, torch.Tensor) else qd
    Md = N if keep_all else max(L.lrm_max_kept(N, qd_host), 1)
    f32, i32 = dict(dtype=torch.float32, device=device), dict(dtype=torch.int32, device=device)
    nan = float("nan")
    wd = dict(dtype=torch.bfloat16 if flags & L.LRM_DW_BF16 else torch.float32, device=device)
    out = dict(dW_gate=torch.full((E, I, H), nan, **wd), dW_up=torch.full((E, I, H), nan, **wd),
               dW_down=torch.full((E, H, I), nan, **wd), dX=torch.full((r.T, H), nan, **f32),
               score=torch.full((max(N, 1),), nan, **f32),
               pos=torch.full((max(N, 1),), -7, **i32),
               offsets=torch.full((E + 1,), -7, **i32),
               score_gate=torch.full((Md,), nan, **f32), score_up=torch.full((Md,), nan, **f32),
               pos_gate=torch.full((Md,), -7, **i32), pos_up=torch.full((Md,), -7, **i32),
               offsets_gate=torch.full((E + 1,), -7, **i32),
               offsets_up=torch.full((E + 1,), -7, **i32),
               dH=torch.full((Md, I), nan, **f32))
    ws = L.lrm_expert_backward(pb, out, ws=ws)
    torch.cuda.synchronize()
    res = {k: v.cpu() for k, v in out.items()}
    res["ws"] = ws
    return res


def judge_swiglu(p: dict, res: dict, keep_all: bool = False, experts=None, tokens=None):
    """Compare one fused SwiGLU result with the oracle (reading R-glu).

    Down stage: scores and kept sets against the pure oracle.  Gate/up stages:
    scores and kept sets against the oracle run on the GPU's own hidden
    gradient u (the chained selection depends on it).  Gradients: the oracle
    re-run on the GPU's kept sets.  ``experts`` samples the experts whose
    weight gradients are formed; ``tokens`` samples dX rows (all if None)."""
    r = p["routing"]
    E, N, H, I = r.E, r.N, p["H"], p["I"]
    tol = TOL[p["dtype"]]
    pos = res["pos"][:N].numpy()
    offs = res["offsets"].numpy().astype(np.int64)
    check_packing(pos, offs, r.expert, E)
    Kd = kept_from_pos(pos, r.expert, E)
    summary = {"kept_down": int(offs[-1])}
    if keep_all:
        assert all(k.size == c for k, c in zip(Kd, r.counts))
    else:
        s64 = O.swiglu_down_scores(p)
        gs = res["score"][:N].numpy().astype(np.float64)
        rel = np.abs(gs - s64) / np.maximum(s64, 1e-300)
        summary["score_down_max_rel"] = float(rel.max()) if N else 0.0
        assert rel.max() < 1e-6 if N else True, rel.max()
        ora_kd = O.select_top_quota(r.expert, s64, p["quota_down"], E)
        summary["ndiff_down"] = check_selection(Kd, ora_kd, s64, r.counts, "down")
    Md = int(offs[-1])
    ex = list(range(E)) if experts is None else list(experts)
    U = res["dH"].numpy()
    kept_g, kept_u = {}, {}
    for e in ex:
        a, b = offs[e], offs[e + 1]
        if keep_all:
            kept_g[e], kept_u[e] = Kd[e], Kd[e]
            continue
        pg = res["pos_gate"].numpy()[a:b]
        pu = res["pos_up"].numpy()[a:b]
        kept_g[e], kept_u[e] = Kd[e][pg >= 0], Kd[e][pu >= 0]
    if not keep_all:
        # gate/up selections judged on the GPU's own u (upcast to fp64)
        uo = {e: U[offs[e]:offs[e + 1]] for e in ex}
        chk = O.swiglu_reference(p, experts=ex, u_override=uo, kept={"down": Kd}, grads=False)
        for name, kg, key in (("gate", kept_g, "K_gate"), ("up", kept_u, "K_up")):
            sk = "s_" + name
            nd = 0
            for e in ex:
                kd = Kd[e]
                gpu_s = res["score_" + name].numpy()[offs[e]:offs[e + 1]].astype(np.float64)
                ref_s = chk[sk][e]
                if kd.size:
                    rel = np.abs(gpu_s - ref_s) / np.maximum(ref_s, 1e-300)
                    assert rel.max() < 2e-6, (name, e, rel.max())
                full = np.zeros(N)
                full[kd] = ref_s
                cnt = np.bincount(r.expert[kd], minlength=E)
                nd += check_selection([kg[e]], [chk[key][e]], full, [cnt[e]], f"{name} e{e}")
            summary["ndiff_" + name] = nd
            o2 = res["offsets_" + name].numpy().astype(np.int64)
            for e in ex:
                assert o2[e + 1] - o2[e] == kg[e].size
    # gradients on the GPU's kept sets, expert by expert
    ref = O.swiglu_reference(p, experts=ex, kept={"down": Kd, "gate": kept_g, "up": kept_u})
    errs = {}
    sizes = {"dW_down": {e: Kd[e].size for e in ex}, "dW_gate": {e: kept_g[e].size for e in ex},
             "dW_up": {e: kept_u[e].size for e in ex}}
    for name in ("dW_down", "dW_gate", "dW_up"):
        got = {e: res[name][e].float().numpy() for e in ex}
        errs[name + "_worst_expert"] = check_per_expert(name, got, ref[name], ex, sizes[name],
                                                        tol)
        errs[name] = rel_fro(np.stack([got[e] for e in ex]),
                             np.stack([ref[name][e] for e in ex]))
    for e in range(E):
        if offs[e + 1] == offs[e]:
            assert not res["dW_down"][e].any() and not res["dW_gate"][e].any() \
                and not res["dW_up"][e].any(), f"expert {e} kept nothing but dW != 0"
    dX = res["dX"].numpy()
    if experts is None and tokens is None:
        errs["dX"] = rel_fro(dX, ref["dX"])
        errs["dX_worst_block"] = check_row_blocks("dX", dX, ref["dX"], tol)
    else:
        toks = np.asarray(tokens if tokens is not None else np.arange(min(r.T, 16)))
        want = np.zeros((toks.size, H))
        # every down-kept pair of the sampled tokens, with its gate/up decisions
        # read from the GPU's packed-row maps
        row_of = np.full(r.T, -1, np.int64)
        row_of[toks] = np.arange(toks.size)
        qs = np.nonzero((row_of[r.token] >= 0) & (pos >= 0))[0]
        if keep_all:
            ing = inu = np.ones(qs.size, bool)
        else:
            ing = res["pos_gate"].numpy()[pos[qs]] >= 0
            inu = res["pos_up"].numpy()[pos[qs]] >= 0
        if qs.size:
            np.add.at(want, row_of[r.token[qs]], O.swiglu_pair_dx(p, qs, ing, inu))
        errs["dX_sampled"] = rel_fro(dX[toks], want)
        errs["dX_worst_block"] = check_row_blocks("dX (sampled tokens)", dX[toks], want, tol)
    summary.update(errs)
    return summary


def judge_linear(p: dict, res: dict, keep_all: bool = False, experts=None):
    """Compare one fused LINEAR result with the oracle.  Returns a summary."""
    r = p["routing"]
    tol = TOL[p["dtype"]]
    s64 = O.linear_scores(p)
    if not keep_all:
        gs = res["score"][: r.N].numpy().astype(np.float64)
        # the GPU key is the fp64 score rounded once to fp32
        np.testing.assert_allclose(gs, s64, rtol=2 ** -23, atol=0)
    q = np.full(r.E, r.N, np.int64) if keep_all else p["quota"]
    ora_kept = O.select_top_quota(r.expert, s64, q, r.E)
    pos = res["pos"][: r.N].numpy()
    gpu_kept = kept_from_pos(pos, r.expert, r.E)
    ndiff = check_selection(gpu_kept, ora_kept, s64, r.counts, "linear")
    check_packing(pos, res["offsets"].numpy(), r.expert, r.E)
    dW_ref, dX_ref = O.linear_backward(p, gpu_kept, experts)
    dW = res["dW"].float().numpy()
    ex = sorted(dW_ref)
    worst_w = check_per_expert("dW", dW, dW_ref, ex, [k.shape[0] for k in gpu_kept], tol)
    worst_x = check_row_blocks("dX", res["dX"].numpy(), dX_ref, tol)
    e_dw = rel_fro(dW[ex], np.stack([dW_ref[e] for e in ex]))
    e_dx = rel_fro(res["dX"].numpy(), dX_ref)
    return dict(ndiff=ndiff, err_dW=e_dw, err_dX=e_dx, worst_expert_dW=worst_w,
                worst_block_dX=worst_x, kept=int(sum(k.size for k in gpu_kept)))
