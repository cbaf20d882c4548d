"""CPU oracle for the LRM-pruned MoE expert backward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke entry point and the benchmark's CPU-baseline leg
may import this module.  The product path (the HIP library and its binding)
never calls it, and this module imports nothing from the product package.

Everything is computed in float64 on exact upcasts of the inputs (fp32 and bf16
values are exactly representable in fp64), in plain NumPy, in the order the
pages describe the method.  Sources (three web pages on one paper):

  [P1] "LRMoE урезает обратный проход MoE и ускоряет обучение на 21–45%"
       (news.hamidun.com, Russian), section "Что делает LRMoE: полный прямой
       проход, обрезанный обратный" (what LRMoE does) and its bullets
       "Квоты до вычислений" (quotas), "Отбор по метрике LRM" (selection by
       the LRM metric), "Физическое уплотнение" (physical compaction), plus the
       note after the bullets on masking.
  [P2] "LRMoE élague la passe arrière des MoE et accélère l'entraînement de
       21–45%" (news.hamidun.com, French), the same section
       "Ce que fait LRMoE : passe avant complète, passe arrière élaguée".
  [P3] "LRMoE führt eine Nachkalibrierung der Last auf der Nachfrageseite ...
       ein" (ai.mistergeeks.com, German), the paragraph on the two-phase
       design and the "Lastnachkalibrierungs-Metrik".

What the pages fix, restated:
  * A pair is one token -> expert routing choice ([P1] intro).
  * A controller fixes, per expert, how many pairs to keep in the backward,
    for the whole layer call ([P1] bullet "Квоты до вычислений").
  * When the gradient reaches the layer, each pair's contribution to its
    expert's weight update is the outer product of the incoming gradient and
    the saved projection input; its squared norm factorises into squared
    routing weight x squared gradient norm x squared input norm, so no full
    gradient matrix is formed; within the quota the highest-scoring pairs are
    kept ([P1] bullet "Отбор по метрике LRM"; [P3] metric paragraph).
  * Kept gradient and activation rows are packed into dense per-expert blocks,
    the products run as variable-size grouped GEMMs without zero padding, and
    the result goes back to the original layout ([P1] bullet
    "Физическое уплотнение").
  * Masking dropped rows in full-size tensors is equivalent but saves nothing
    ([P1] note after the bullets).
  * Dropped pairs' gradient contributions are discarded; the metric is a
    per-projection estimate ([P1] section "Что показали эксперименты и где
    подвох").

Readings where the pages are silent (each also listed in the design notes):
  R-g   the incoming gradient g of a pair is unscaled; the contribution to
        dW_e is (w g) x^T, so the score is w^2 |g|^2 |x|^2.
  R-tie candidates are ordered by score descending, then pair index
        ascending; the first min(q_e, n_e) are kept.
  R-drop a dropped pair contributes to neither dW nor dX.
  R-glu SwiGLU runs down -> gate/up; the down stage's dropped pairs carry no
        gradient further, so the gate/up candidates of expert e are the pairs
        kept by its down stage; gate and up each have their own score, quota
        and kept set.

Every function here is pinned by tests against something other than itself
(closed forms, brute force, torch.autograd in fp64, hand-worked fixtures).
"""

from __future__ import annotations

import numpy as np

TOKEN = "token"
PAIR = "pair"


# ------------------------------------------------------------------ helpers

def f64(a) -> np.ndarray:
    """Exact float64 copy of a NumPy array or a CPU torch tensor."""
    if hasattr(a, "detach"):  # torch tensor (bf16 has no NumPy dtype)
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def pair_rows(mat, rows: str, token: np.ndarray, pairs: np.ndarray) -> np.ndarray:
    """fp64 rows of ``mat`` seen by the given pairs: row token[p] or row p."""
    idx = token[pairs] if rows == TOKEN else pairs
    if hasattr(mat, "detach"):
        import torch
        return mat[torch.as_tensor(idx, dtype=torch.long)].to(torch.float64).numpy()
    return np.asarray(mat[idx], dtype=np.float64)


def _chunks(n: int, chunk: int, fn) -> None:
    """Apply fn(r0, r1) to row ranges; ranges are independent, so they may run
    on several host threads without changing any result."""
    import concurrent.futures as cf
    import os
    ranges = [(r0, min(r0 + chunk, n)) for r0 in range(0, n, chunk)]
    if len(ranges) <= 1:
        for a, b in ranges:
            fn(a, b)
        return
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda ab: fn(*ab), ranges))


def row_sumsq(mat, chunk: int = 8192) -> np.ndarray:
    """Sum of squares of every row, in fp64 (rows visited in chunks)."""
    out = np.empty(mat.shape[0], dtype=np.float64)

    def work(r0, r1):
        m = f64(mat[r0:r1])
        out[r0:r1] = (m * m).sum(axis=1)
    _chunks(mat.shape[0], chunk, work)
    return out


# ---------------------------------------------------------------- the score

def lrm_score(w: np.ndarray, g_sumsq: np.ndarray, x_sumsq: np.ndarray) -> np.ndarray:
    """LRM score of each pair: w^2 * |g|^2 * |x|^2 ([P1] bullet
    "Отбор по метрике LRM"; [P2] "Sélection par la métrique LRM").  This is
    the squared Frobenius norm of the pair's weight-gradient contribution
    (w g) x^T, without forming it."""
    w = np.asarray(w, dtype=np.float64)
    return (w * w) * g_sumsq * x_sumsq


# ------------------------------------------------------------ the selection

def select_top_quota(expert: np.ndarray, score: np.ndarray, quota: np.ndarray, E: int,
                     candidates: np.ndarray | None = None) -> list[np.ndarray]:
    """Per expert, keep the min(q_e, n_e) highest-scoring candidates
    ([P1] bullets "Квоты до вычислений" and "Отбор по метрике LRM").

    ``candidates`` restricts the candidate pairs (default: all pairs).  Order:
    score descending, ties by pair index ascending (reading R-tie).  Returns,
    per expert, the kept pair indices in ascending order."""
    expert = np.asarray(expert)
    score = np.asarray(score, dtype=np.float64)
    quota = np.asarray(quota)
    if np.any(quota < 0):
        raise ValueError("negative quota")
    pool = np.arange(expert.shape[0]) if candidates is None else np.sort(candidates)
    kept = []
    for e in range(E):
        cand = pool[expert[pool] == e]
        m = min(int(quota[e]), cand.shape[0])
        order = np.lexsort((cand, -score[cand]))  # primary -score, then index
        kept.append(np.sort(cand[order[:m]]))
    return kept


def pack(kept: list[np.ndarray], N: int):
    """Dense per-expert packing of the kept pairs ([P1] bullet
    "Физическое уплотнение"): expert blocks back to back, no padding, pairs
    ascending inside a block.  Returns (offsets[E+1], kept_list[M], pos[N])
    with pos[p] the packed row of p or -1."""
    sizes = np.array([k.shape[0] for k in kept], dtype=np.int64)
    offsets = np.zeros(len(kept) + 1, dtype=np.int64)
    np.cumsum(sizes, out=offsets[1:])
    kept_list = np.concatenate(kept).astype(np.int64) if kept else np.zeros(0, np.int64)
    pos = np.full(N, -1, dtype=np.int64)
    pos[kept_list] = np.arange(kept_list.shape[0])
    return offsets, kept_list, pos


def threshold(score: np.ndarray, kept_e: np.ndarray, n_e: int) -> float | None:
    """The M_e-th largest score of an expert (None when nothing or everything
    is kept): the boundary a selection decision is taken against."""
    m = kept_e.shape[0]
    if m == 0 or m == n_e:
        return None
    return float(np.min(np.asarray(score, np.float64)[kept_e]))


# ------------------------------------------------------ LINEAR projection

def linear_scores(p: dict) -> np.ndarray:
    """Scores of every pair of a single projection: g from G, x from X."""
    r = p["routing"]
    gs = row_sumsq(p["G"])
    xs = row_sumsq(p["X"])
    g2 = gs[r.token] if p["G_rows"] == TOKEN else gs
    x2 = xs[r.token] if p["X_rows"] == TOKEN else xs
    return lrm_score(r.weight, g2, x2)


def linear_dW_expert(p: dict, e: int, kept_e: np.ndarray) -> np.ndarray:
    """dW_e = sum over kept pairs of (w g) x^T, shape [d_out, d_in]; zero if
    nothing is kept (reading R-drop)."""
    r = p["routing"]
    if kept_e.shape[0] == 0:
        return np.zeros((p["d_out"], p["d_in"]))
    g = pair_rows(p["G"], p["G_rows"], r.token, kept_e)
    x = pair_rows(p["X"], p["X_rows"], r.token, kept_e)
    w = r.weight[kept_e].astype(np.float64)
    return g.T @ (w[:, None] * x)


def linear_dx_pairs(p: dict, e: int, kept_e: np.ndarray) -> np.ndarray:
    """Input gradient of every kept pair of expert e: w W_e^T g, rows [M_e, d_in]."""
    r = p["routing"]
    if kept_e.shape[0] == 0:
        return np.zeros((0, p["d_in"]))
    g = pair_rows(p["G"], p["G_rows"], r.token, kept_e)
    We = f64(p["W"][e])
    w = r.weight[kept_e].astype(np.float64)
    return w[:, None] * (g @ We)


def linear_backward(p: dict, kept: list[np.ndarray], experts=None):
    """dW (per listed expert) and dX in the layout of X (TOKEN: sum over the
    token's pairs, zero rows where nothing is kept; PAIR: one row per pair,
    zero for dropped pairs) -- the result back in the original layout
    ([P1] bullet "Физическое уплотнение")."""
    r = p["routing"]
    E = r.E
    experts = range(E) if experts is None else experts
    dW = {e: linear_dW_expert(p, e, kept[e]) for e in experts}
    rows = r.T if p["X_rows"] == TOKEN else r.N
    dX = np.zeros((rows, p["d_in"]))
    for e in range(E):
        K = kept[e]
        if K.shape[0] == 0:
            continue
        dx = linear_dx_pairs(p, e, K)
        if p["X_rows"] == TOKEN:
            np.add.at(dX, r.token[K], dx)
        else:
            dX[K] = dx
    return dW, dX


def linear_backward_masked(p: dict, mask: np.ndarray):
    """The same gradients computed over full-size tensors with dropped rows
    multiplied by zero (the alternative the pages note gains nothing)."""
    r = p["routing"]
    allp = np.arange(r.N)
    g = pair_rows(p["G"], p["G_rows"], r.token, allp)
    x = pair_rows(p["X"], p["X_rows"], r.token, allp)
    wm = r.weight.astype(np.float64) * mask.astype(np.float64)
    dW = np.zeros((r.E, p["d_out"], p["d_in"]))
    dxp = np.zeros((r.N, p["d_in"]))
    for e in range(r.E):
        sel = (r.expert == e).astype(np.float64)
        dW[e] = (g * (wm * sel)[:, None]).T @ x
        dxp += (wm * sel)[:, None] * (g @ f64(p["W"][e]))
    if p["X_rows"] == TOKEN:
        dX = np.zeros((r.T, p["d_in"]))
        np.add.at(dX, r.token, dxp)
    else:
        dX = dxp
    return dW, dX


def linear_reference(p: dict, keep_all: bool = False, experts=None) -> dict:
    """Whole LINEAR backward: scores, kept sets, packing, dW, dX."""
    r = p["routing"]
    s = linear_scores(p)
    q = np.full(r.E, r.N, dtype=np.int64) if keep_all else p["quota"]
    kept = select_top_quota(r.expert, s, q, r.E)
    offsets, kept_list, pos = pack(kept, r.N)
    dW, dX = linear_backward(p, kept, experts)
    return dict(score=s, kept=kept, offsets=offsets, kept_list=kept_list, pos=pos,
                dW=dW, dX=dX)


# ------------------------------------------------------- SwiGLU expert MLP

def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def silu(a):
    """silu(a) = a * sigmoid(a)."""
    return a * sigmoid(a)


def dsilu(a):
    """d silu / da = sigmoid(a) * (1 + a * (1 - sigmoid(a)))."""
    s = sigmoid(a)
    return s * (1.0 + a * (1.0 - s))


def swiglu_down_scores(p: dict) -> np.ndarray:
    """Down projection: input h = silu(a) * b (per pair, from the saved gate
    and up pre-activations), incoming gradient g = G[token]."""
    r = p["routing"]
    gs = row_sumsq(p["G"])[r.token]
    hs = np.empty(r.N)

    def work(r0, r1):
        h = silu(f64(p["A"][r0:r1])) * f64(p["B"][r0:r1])
        hs[r0:r1] = (h * h).sum(axis=1)
    _chunks(r.N, 8192, work)
    return lrm_score(r.weight, gs, hs)


def swiglu_expert_down(p: dict, e: int, kd: np.ndarray):
    """For the down-kept pairs of expert e: dW_down_e [H, I] and the unscaled
    hidden gradient u = W_down_e^T g of each pair, rows [M_e, I]."""
    r = p["routing"]
    H, I = p["H"], p["I"]
    if kd.shape[0] == 0:
        return np.zeros((H, I)), np.zeros((0, I))
    g = pair_rows(p["G"], TOKEN, r.token, kd)
    a = f64(p["A"][kd])
    b = f64(p["B"][kd])
    h = silu(a) * b
    w = r.weight[kd].astype(np.float64)
    dWd = g.T @ (w[:, None] * h)
    u = g @ f64(p["W_down"][e])
    return dWd, u


def swiglu_gate_up_grads(p: dict, kd: np.ndarray, u: np.ndarray):
    """Unscaled gradients at the gate and up pre-activations of the down-kept
    pairs: ga = u * b * silu'(a), gb = u * silu(a)."""
    a = f64(p["A"][kd])
    b = f64(p["B"][kd])
    return u * b * dsilu(a), u * silu(a)


def swiglu_reference(p: dict, experts=None, keep_all: bool = False,
                     u_override: dict | None = None, kept: dict | None = None,
                     grads: bool = True) -> dict:
    """The SwiGLU expert backward (reading R-glu), expert by expert.

    ``experts`` limits which experts' weight gradients and pair gradients are
    formed (all by default); kept sets of the down stage are always complete.
    ``u_override[e]`` replaces the hidden gradient of expert e's down-kept
    pairs (used to judge the second selection on another implementation's
    own intermediate values).  ``kept`` may hold any of "down" (a list per
    expert), "gate" and "up" (dicts by expert): given kept sets replace the
    corresponding selections (the same arithmetic re-run on another
    implementation's choices; when "down" is given no down scores are formed).
    ``grads=False`` stops after the selections (scores and kept sets only).
    Returns kept sets, scores, dW per expert and, when every expert is
    formed, dX [T, H]."""
    r = p["routing"]
    E = r.E
    big = np.full(E, r.N, dtype=np.int64)
    qd = big if keep_all else p["quota_down"]
    qg = big if keep_all else p["quota_gate"]
    qu = big if keep_all else p["quota_up"]
    kept = kept or {}
    if "down" not in kept:
        s_down = swiglu_down_scores(p)
        K_down = select_top_quota(r.expert, s_down, qd, E)
    else:
        s_down = None
        K_down = [np.sort(np.asarray(k, dtype=np.int64)) for k in kept["down"]]
    x2 = row_sumsq(p["X"])
    experts = list(range(E)) if experts is None else list(experts)
    out = dict(s_down=s_down, K_down=K_down, K_gate={}, K_up={}, s_gate={}, s_up={},
               dW_down={}, dW_gate={}, dW_up={}, dx_pairs={})
    H = p["H"]
    for e in experts:
        kd = K_down[e]
        if u_override is not None and e in u_override:
            u = np.asarray(u_override[e], dtype=np.float64)
            dWd = swiglu_expert_down(p, e, kd)[0] if grads else None
        else:
            dWd, u = swiglu_expert_down(p, e, kd)
        ga, gb = swiglu_gate_up_grads(p, kd, u)
        w = r.weight[kd].astype(np.float64)
        sg = lrm_score(w, (ga * ga).sum(axis=1), x2[r.token[kd]])
        su = lrm_score(w, (gb * gb).sum(axis=1), x2[r.token[kd]])
        # candidates of the gate/up selections: this expert's down-kept pairs
        s_full_g = np.zeros(r.N)
        s_full_g[kd] = sg
        s_full_u = np.zeros(r.N)
        s_full_u[kd] = su
        if "gate" in kept:
            Kg = np.sort(np.asarray(kept["gate"][e], dtype=np.int64))
        else:
            Kg = select_top_quota(r.expert, s_full_g, qg, E, candidates=kd)[e]
        if "up" in kept:
            Ku = np.sort(np.asarray(kept["up"][e], dtype=np.int64))
        else:
            Ku = select_top_quota(r.expert, s_full_u, qu, E, candidates=kd)[e]
        out["K_gate"][e], out["K_up"][e] = Kg, Ku
        out["s_gate"][e], out["s_up"][e] = sg, su
        if not grads:
            continue
        row = {pp: i for i, pp in enumerate(kd.tolist())}
        ig = np.array([row[pp] for pp in Kg.tolist()], dtype=np.int64)
        iu = np.array([row[pp] for pp in Ku.tolist()], dtype=np.int64)
        xg = pair_rows(p["X"], TOKEN, r.token, Kg) if Kg.size else np.zeros((0, H))
        xu = pair_rows(p["X"], TOKEN, r.token, Ku) if Ku.size else np.zeros((0, H))
        wg = r.weight[Kg].astype(np.float64)
        wu = r.weight[Ku].astype(np.float64)
        out["dW_down"][e] = dWd
        out["dW_gate"][e] = ga[ig].T @ (wg[:, None] * xg) if Kg.size else np.zeros((p["I"], H))
        out["dW_up"][e] = gb[iu].T @ (wu[:, None] * xu) if Ku.size else np.zeros((p["I"], H))
        dx = np.zeros((kd.shape[0], H))
        if Kg.size:
            dx[ig] += wg[:, None] * (ga[ig] @ f64(p["W_gate"][e]))
        if Ku.size:
            dx[iu] += wu[:, None] * (gb[iu] @ f64(p["W_up"][e]))
        out["dx_pairs"][e] = (kd, dx)
    if grads and len(experts) == E:
        dX = np.zeros((r.T, H))
        for e in range(E):
            kd, dx = out["dx_pairs"][e]
            if kd.size:
                np.add.at(dX, r.token[kd], dx)
        out["dX"] = dX
    return out


def swiglu_pair_dx(p: dict, pairs, in_gate, in_up) -> np.ndarray:
    """Input-gradient row of each listed down-kept pair q (token t, expert e):
    w_q (1[q kept by gate] ga_q W_gate_e + 1[q kept by up] gb_q W_up_e), with
    u = W_down_e^T g_t, ga = u * b * silu'(a), gb = u * silu(a).  The pairs of
    one expert are formed together (each row is independent of the others)."""
    r = p["routing"]
    pairs = np.asarray(pairs, dtype=np.int64)
    in_gate = np.asarray(in_gate, dtype=bool)
    in_up = np.asarray(in_up, dtype=bool)
    out = np.zeros((pairs.shape[0], p["H"]))
    for e in np.unique(r.expert[pairs]) if pairs.size else []:
        sel = np.nonzero(r.expert[pairs] == e)[0]
        q = pairs[sel]
        g = pair_rows(p["G"], TOKEN, r.token, q)
        u = g @ f64(p["W_down"][e])
        ga, gb = swiglu_gate_up_grads(p, q, u)
        dx = np.zeros((q.shape[0], p["H"]))
        mg, mu = in_gate[sel], in_up[sel]
        if mg.any():
            dx[mg] += ga[mg] @ f64(p["W_gate"][e])
        if mu.any():
            dx[mu] += gb[mu] @ f64(p["W_up"][e])
        out[sel] = r.weight[q].astype(np.float64)[:, None] * dx
    return out
