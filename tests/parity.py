"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and judge it against the fp64 oracle.

Parity rule for selections (several kept sets can be correct when scores tie
or nearly tie): the GPU keeps exactly M_e = min(q_e, n_e) pairs per expert,
and every pair in the symmetric difference with the oracle's kept set has an
oracle score within 1e-6 relative of the expert's threshold tau_e (the
oracle's M_e-th largest score).  Gradients are then compared with the oracle
re-run on the GPU's kept sets, by relative Frobenius error: 1e-5 for fp32
inputs, 2e-2 for bf16 inputs with fp32 accumulation.  Experts with nothing
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
    out = dict(dW=torch.full((r.E, p["d_out"], p["d_in"]), float("nan"), **f32),
               dX=torch.full((rows, p["d_in"]), float("nan"), **f32),
               score=torch.full((max(r.N, 1),), float("nan"), **f32),
               pos=torch.full((max(r.N, 1),), -7, **i32),
               offsets=torch.full((r.E + 1,), -7, **i32))
    ws = L.lrm_expert_backward(pb, out, ws=ws)
    torch.cuda.synchronize()
    res = {k: v.cpu() for k, v in out.items()}
    res["ws"] = ws
    return res


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
    dW = res["dW"].numpy()
    errs = []
    for e in dW_ref:
        if gpu_kept[e].shape[0] == 0:
            assert not np.any(dW[e]), f"expert {e} kept nothing but dW != 0"
    ref = np.stack([dW_ref[e] for e in sorted(dW_ref)])
    got = dW[sorted(dW_ref)]
    e_dw = rel_fro(got, ref)
    e_dx = rel_fro(res["dX"].numpy(), dX_ref)
    assert e_dw <= tol, f"dW rel err {e_dw}"
    assert e_dx <= tol, f"dX rel err {e_dx}"
    zero_rows = ~np.any(dX_ref != 0, axis=1)
    assert not np.any(res["dX"].numpy()[zero_rows]), "rows without kept pairs must be 0"
    return dict(ndiff=ndiff, err_dW=e_dw, err_dX=e_dx, kept=int(sum(k.size for k in gpu_kept)))
