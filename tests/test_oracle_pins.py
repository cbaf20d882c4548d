"""Pins of the CPU oracle against things other than itself.

* hand-worked fixtures under tests/golden/ (closed forms, exact dyadic values);
* per-pair torch.autograd in fp64: each pair's weight-gradient contribution is
  formed explicitly as a full matrix, so its squared Frobenius norm is the
  brute-force score, a Python sort of those norms is the brute-force kept set,
  and the sum of the kept contributions is the brute-force weight gradient;
* invariants: keep-all equals the unpruned autograd backward, quota 0 gives
  zeros, masked full-size equals compacted, additivity over disjoint kept
  sets, token permutation, score scaling.
"""

import json
import os
import types

import numpy as np
import pytest
import torch

from oracle import lrm_oracle as O
from pruned_expert_backward_lrm_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _routing(d):
    tok = np.array(d["token"], np.int32)
    ex = np.array(d["expert"], np.int32)
    w = np.array(d["weight"], np.float32)
    return types.SimpleNamespace(T=d["T"], E=d["E"], N=len(tok), token=tok, expert=ex,
                                 weight=w, counts=np.bincount(ex, minlength=d["E"]))


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


# ------------------------------------------------------------------ golden

def test_golden_linear_hand_example():
    d = json.load(open(os.path.join(GOLD, "hand_linear.json")))
    p = dict(routing=_routing(d), X=np.array(d["X"], float), G=np.array(d["G"], float),
             W=np.array(d["W"], float), X_rows=d["X_rows"], G_rows=d["G_rows"],
             d_in=d["d_in"], d_out=d["d_out"], quota=np.array(d["quota"]))
    ref = O.linear_reference(p)
    ex = d["expect"]
    assert ref["score"].tolist() == ex["score"]
    assert [k.tolist() for k in ref["kept"]] == ex["kept"]
    assert ref["offsets"].tolist() == ex["offsets"]
    assert ref["pos"].tolist() == ex["pos"]
    assert np.array_equal(np.stack([ref["dW"][e] for e in range(2)]), np.array(ex["dW"]))
    assert np.array_equal(ref["dX"], np.array(ex["dX"]))


def test_golden_swiglu_hand_example():
    d = json.load(open(os.path.join(GOLD, "hand_swiglu.json")))
    p = dict(routing=_routing(d), H=d["H"], I=d["I"],
             **{k: np.array(d[k], float) for k in ("X", "G", "A", "B", "W_gate", "W_up", "W_down")},
             **{k: np.array(d[k]) for k in ("quota_down", "quota_gate", "quota_up")})
    ref = O.swiglu_reference(p)
    ex = d["expect"]
    assert ref["s_down"].tolist() == ex["s_down"]
    assert [k.tolist() for k in ref["K_down"]] == ex["K_down"]
    assert [ref["K_gate"][0].tolist()] == ex["K_gate"]
    assert [ref["K_up"][0].tolist()] == ex["K_up"]
    assert ref["s_gate"][0].tolist() == ex["s_gate"]
    assert ref["s_up"][0].tolist() == ex["s_up"]
    assert ref["dW_down"][0].tolist() == ex["dW_down"][0]
    assert ref["dW_gate"][0].tolist() == ex["dW_gate"][0]
    assert ref["dW_up"][0].tolist() == ex["dW_up"][0]
    assert ref["dX"].tolist() == ex["dX"]


# -------------------------------------------- per-pair autograd (LINEAR)

def _linear_problem(T=24, E=3, k=2, d_in=6, d_out=5, x_rows="token", g_rows="pair", seed=0,
                    quota=None):
    p = synth.make_linear(T, E, k, d_in, d_out, dtype="f32", x_rows=x_rows, g_rows=g_rows,
                          seed=seed, quota=quota, g_std=1.0)
    return p


def _linear_pair_terms(p):
    """For every pair p: (dL_p/dW_e as a full matrix, dL_p/dx row), where the
    pair's loss term is L_p = w_p <g_p, W_e x_p> (g_p the incoming gradient
    at the pair's projection output)."""
    r = p["routing"]
    W = torch.tensor(O.f64(p["W"]))
    X = torch.tensor(O.f64(p["X"]))
    G = torch.tensor(O.f64(p["G"]))
    out = []
    for q in range(r.N):
        Wl = W.clone().requires_grad_(True)
        Xl = X.clone().requires_grad_(True)
        xr = int(r.token[q]) if p["X_rows"] == "token" else q
        gr = int(r.token[q]) if p["G_rows"] == "token" else q
        e = int(r.expert[q])
        L = float(r.weight[q]) * torch.dot(G[gr], Wl[e] @ Xl[xr])
        L.backward()
        out.append((Wl.grad[e].numpy().copy(), Xl.grad.numpy().copy()))
    return out


def _bruteforce_kept(norms, expert, quota, E, cand=None):
    kept = []
    N = len(norms)
    pool = range(N) if cand is None else sorted(cand)
    for e in range(E):
        c = [q for q in pool if expert[q] == e]
        m = min(int(quota[e]), len(c))
        kept.append(sorted(sorted(c, key=lambda q: (-norms[q], q))[:m]))
    return kept


@pytest.mark.parametrize("x_rows,g_rows", [("token", "pair"), ("pair", "token"),
                                           ("token", "token"), ("pair", "pair")])
def test_linear_against_per_pair_autograd(x_rows, g_rows):
    p = _linear_problem(x_rows=x_rows, g_rows=g_rows, seed=3)
    r = p["routing"]
    terms = _linear_pair_terms(p)
    # score: squared Frobenius norm of the explicitly formed contribution
    norms = [float((c * c).sum()) for c, _ in terms]
    s = O.linear_scores(p)
    np.testing.assert_allclose(s, norms, rtol=1e-12, atol=0)
    # selection: Python sort of the brute-force norms
    kept = O.select_top_quota(r.expert, s, p["quota"], r.E)
    bf = _bruteforce_kept(norms, r.expert, p["quota"], r.E)
    assert [k.tolist() for k in kept] == bf
    # gradients: sum of the kept pairs' contributions
    dW, dX = O.linear_backward(p, kept)
    kept_all = [q for kk in bf for q in kk]
    for e in range(r.E):
        want = sum((terms[q][0] for q in bf[e]), np.zeros((p["d_out"], p["d_in"])))
        assert _rel(dW[e], want) < 1e-12
    want_dx = sum((terms[q][1] for q in kept_all), np.zeros_like(dX))
    assert _rel(dX, want_dx) < 1e-12


def test_linear_keep_all_is_unpruned_autograd():
    """Quota >= count reproduces the ordinary dense backward of the layer."""
    p = _linear_problem(T=20, E=4, k=2, seed=5, quota=lambda c: c + 3)
    r = p["routing"]
    W = torch.tensor(O.f64(p["W"]), requires_grad=True)
    X = torch.tensor(O.f64(p["X"]), requires_grad=True)
    G = torch.tensor(O.f64(p["G"]))
    xs = X[torch.as_tensor(r.token, dtype=torch.long)]
    We = W[torch.as_tensor(r.expert, dtype=torch.long)]
    y = torch.tensor(r.weight, dtype=torch.float64)[:, None] * torch.einsum("poi,pi->po", We, xs)
    (G * y).sum().backward()
    ref = O.linear_reference(p)
    assert all(k.shape[0] == c for k, c in zip(ref["kept"], r.counts))
    for e in range(r.E):
        assert _rel(ref["dW"][e], W.grad[e].numpy()) < 1e-12
    assert _rel(ref["dX"], X.grad.numpy()) < 1e-12


def test_quota_zero_gives_zeros():
    p = _linear_problem(seed=7, quota=lambda c: 0 * c)
    ref = O.linear_reference(p)
    assert all(k.shape[0] == 0 for k in ref["kept"])
    assert all(not ref["dW"][e].any() for e in ref["dW"])
    assert not ref["dX"].any()
    assert (ref["pos"] == -1).all() and ref["offsets"][-1] == 0


def test_negative_quota_rejected():
    p = _linear_problem(seed=7)
    r = p["routing"]
    with pytest.raises(ValueError):
        O.select_top_quota(r.expert, O.linear_scores(p), -np.ones(r.E, np.int64), r.E)


# ------------------------------------------------------------- selection

def test_select_top_q_property_and_ties():
    rng = np.random.default_rng(11)
    N, E = 400, 5
    expert = rng.integers(0, E, N).astype(np.int32)
    # heavy ties: only 7 distinct score values
    score = rng.integers(0, 7, N).astype(np.float64)
    quota = rng.integers(0, 120, E)
    kept = O.select_top_quota(expert, score, quota, E)
    bf = _bruteforce_kept(score.tolist(), expert, quota, E)
    assert [k.tolist() for k in kept] == bf
    for e in range(E):
        cand = np.nonzero(expert == e)[0]
        K = set(kept[e].tolist())
        assert len(K) == min(quota[e], cand.size)
        drop = [q for q in cand if q not in K]
        if K and drop:
            lo = min(score[q] for q in K)
            assert lo >= max(score[q] for q in drop)
            # among the threshold ties, the kept ones have the lowest indices
            tie_k = [q for q in K if score[q] == lo]
            tie_d = [q for q in drop if score[q] == lo]
            if tie_d:
                assert max(tie_k) < min(tie_d)


def test_select_duplicated_rows_tie_break():
    """Identical pairs (same rows, same weight) tie exactly: lower index wins."""
    d = json.load(open(os.path.join(GOLD, "hand_linear.json")))
    r = _routing(dict(d, token=[0, 0, 1, 1], expert=[0, 0, 0, 0], weight=[0.5] * 4))
    X = np.array([[1.0, 2.0], [1.0, 2.0]])
    p = dict(routing=r, X=X, G=np.ones((4, 2)), W=np.zeros((2, 2, 2)), X_rows="token",
             G_rows="pair", d_in=2, d_out=2, quota=np.array([3, 0]))
    ref = O.linear_reference(p)
    assert ref["score"].tolist() == [2.5] * 4
    assert ref["kept"][0].tolist() == [0, 1, 2]


def test_score_scaling_invariance():
    p = _linear_problem(T=64, E=4, seed=13)
    r = p["routing"]
    s = O.linear_scores(p)
    p2 = dict(p, G=p["G"] * 4.0)
    s2 = O.linear_scores(p2)
    np.testing.assert_array_equal(s2, 16.0 * s)
    k1 = O.select_top_quota(r.expert, s, p["quota"], r.E)
    k2 = O.select_top_quota(r.expert, s2, p["quota"], r.E)
    assert all(np.array_equal(a, b) for a, b in zip(k1, k2))


# ------------------------------------------------------------ invariants

def test_masked_equals_compacted():
    p = _linear_problem(T=48, E=4, seed=17)
    r = p["routing"]
    ref = O.linear_reference(p)
    mask = ref["pos"] >= 0
    dWm, dXm = O.linear_backward_masked(p, mask)
    for e in range(r.E):
        assert _rel(ref["dW"][e], dWm[e]) < 1e-12
    assert _rel(ref["dX"], dXm) < 1e-12


def test_additivity_over_disjoint_kept_sets():
    p = _linear_problem(T=48, E=3, seed=19, quota=lambda c: c)
    r = p["routing"]
    full = O.select_top_quota(r.expert, O.linear_scores(p), p["quota"], r.E)
    k1 = [k[::2] for k in full]
    k2 = [k[1::2] for k in full]
    dW, dX = O.linear_backward(p, full)
    dW1, dX1 = O.linear_backward(p, k1)
    dW2, dX2 = O.linear_backward(p, k2)
    for e in range(r.E):
        assert _rel(dW1[e] + dW2[e], dW[e]) < 1e-12
    assert _rel(dX1 + dX2, dX) < 1e-12


def test_token_permutation_permutes_dx():
    p = _linear_problem(T=32, E=3, k=2, seed=23)
    r = p["routing"]
    ref = O.linear_reference(p)
    rng = np.random.default_rng(5)
    perm = rng.permutation(r.T)          # old token t -> new token perm[t]
    inv = np.argsort(perm)
    # rebuild token-major pairs for the permuted token order
    new_pairs = np.concatenate([np.nonzero(r.token == inv[t])[0] for t in range(r.T)])
    r2 = types.SimpleNamespace(T=r.T, E=r.E, N=r.N, token=perm[r.token[new_pairs]].astype(np.int32),
                               expert=r.expert[new_pairs], weight=r.weight[new_pairs],
                               counts=r.counts)
    X2 = np.empty_like(O.f64(p["X"]))
    X2[perm] = O.f64(p["X"])
    p2 = dict(p, routing=r2, X=X2, G=O.f64(p["G"])[new_pairs])
    ref2 = O.linear_reference(p2)
    for e in range(r.E):
        assert _rel(ref2["dW"][e], ref["dW"][e]) < 1e-12
    assert _rel(ref2["dX"][perm], ref["dX"]) < 1e-12


# ------------------------------------------------ per-pair autograd (SwiGLU)

def _swiglu_problem(T=20, E=3, k=2, H=6, I=5, seed=0, quotas=None):
    """Consistent saved activations: A = X W_gate^T, B = X W_up^T."""
    p = synth.make_swiglu(T, E, k, H, I, dtype="f32", seed=seed, quotas=quotas, g_std=1.0)
    r = p["routing"]
    X = O.f64(p["X"])
    Wg, Wu = O.f64(p["W_gate"]), O.f64(p["W_up"])
    A = np.stack([Wg[r.expert[q]] @ X[r.token[q]] for q in range(r.N)])
    B = np.stack([Wu[r.expert[q]] @ X[r.token[q]] for q in range(r.N)])
    return dict(p, X=X, G=O.f64(p["G"]), A=A, B=B, W_gate=Wg, W_up=Wu,
                W_down=O.f64(p["W_down"]))


def _swiglu_pair_terms(p):
    """Per pair q with L_q = w_q <g_t, W_down silu(W_gate x_t) * (W_up x_t)>:
    contributions to dW_down, dW_gate, dW_up, the x-gradient through the gate
    path and through the up path, and dL_q/da_q, dL_q/db_q."""
    r = p["routing"]
    out = []
    for q in range(r.N):
        e, t, w = int(r.expert[q]), int(r.token[q]), float(r.weight[q])
        Wg = torch.tensor(p["W_gate"][e], requires_grad=True)
        Wu = torch.tensor(p["W_up"][e], requires_grad=True)
        Wd = torch.tensor(p["W_down"][e], requires_grad=True)
        xg = torch.tensor(p["X"][t], requires_grad=True)
        xu = torch.tensor(p["X"][t], requires_grad=True)
        a = Wg @ xg
        b = Wu @ xu
        a.retain_grad()
        b.retain_grad()
        h = torch.nn.functional.silu(a) * b
        L = w * torch.dot(torch.tensor(p["G"][t]), Wd @ h)
        L.backward()
        out.append(dict(down=Wd.grad.numpy().copy(), gate=Wg.grad.numpy().copy(),
                        up=Wu.grad.numpy().copy(), xg=xg.grad.numpy().copy(),
                        xu=xu.grad.numpy().copy(), da=a.grad.numpy().copy(),
                        db=b.grad.numpy().copy()))
    return out


@pytest.mark.parametrize("variant", ["same", "second_selection"])
def test_swiglu_against_per_pair_autograd(variant):
    if variant == "same":
        quotas = (lambda c: c // 2, lambda c: c // 2, lambda c: c // 2)
    else:
        quotas = (lambda c: (3 * c) // 4, lambda c: (3 * c) // 8, lambda c: c // 4)
    p = _swiglu_problem(seed=29 if variant == "same" else 31, quotas=quotas)
    r = p["routing"]
    terms = _swiglu_pair_terms(p)
    ref = O.swiglu_reference(p)
    # down scores = squared Frobenius norms of the per-pair down contributions
    nd = [float((t["down"] ** 2).sum()) for t in terms]
    np.testing.assert_allclose(ref["s_down"], nd, rtol=1e-12, atol=0)
    Kd = _bruteforce_kept(nd, r.expert, p["quota_down"], r.E)
    assert [k.tolist() for k in ref["K_down"]] == Kd
    dX = np.zeros((r.T, p["H"]))
    for e in range(r.E):
        kd = Kd[e]
        ng = {q: float((terms[q]["gate"] ** 2).sum()) for q in kd}
        nu = {q: float((terms[q]["up"] ** 2).sum()) for q in kd}
        np.testing.assert_allclose(ref["s_gate"][e], [ng[q] for q in kd], rtol=1e-12, atol=0)
        np.testing.assert_allclose(ref["s_up"][e], [nu[q] for q in kd], rtol=1e-12, atol=0)
        full_g = np.zeros(r.N)
        full_u = np.zeros(r.N)
        for q in kd:
            full_g[q], full_u[q] = ng[q], nu[q]
        Kg = _bruteforce_kept(full_g, r.expert, p["quota_gate"], r.E, cand=kd)[e]
        Ku = _bruteforce_kept(full_u, r.expert, p["quota_up"], r.E, cand=kd)[e]
        assert ref["K_gate"][e].tolist() == Kg
        assert ref["K_up"][e].tolist() == Ku
        zero = lambda s: np.zeros_like(terms[0][s]) if e == r.expert[0] else None
        for name, K in (("down", kd), ("gate", Kg), ("up", Ku)):
            want = sum((terms[q][name] for q in K), np.zeros_like(ref["dW_" + name][e]))
            assert _rel(ref["dW_" + name][e], want) < 1e-12
        for q in Kg:
            dX[r.token[q]] += terms[q]["xg"]
        for q in Ku:
            dX[r.token[q]] += terms[q]["xu"]
        # the gate/up pre-activation gradients: dL/da = w * ga, dL/db = w * gb
        kd_arr = np.array(kd, dtype=np.int64)
        if kd:
            _, u = O.swiglu_expert_down(p, e, kd_arr)
            ga, gb = O.swiglu_gate_up_grads(p, kd_arr, u)
            w = r.weight[kd_arr].astype(np.float64)[:, None]
            assert _rel(w * ga, np.stack([terms[q]["da"] for q in kd])) < 1e-12
            assert _rel(w * gb, np.stack([terms[q]["db"] for q in kd])) < 1e-12
    assert _rel(ref["dX"], dX) < 1e-12


def test_swiglu_keep_all_is_unpruned_autograd():
    p = _swiglu_problem(seed=37, quotas=(lambda c: c, lambda c: c + 1, lambda c: c + 2))
    r = p["routing"]
    Wg = torch.tensor(p["W_gate"], requires_grad=True)
    Wu = torch.tensor(p["W_up"], requires_grad=True)
    Wd = torch.tensor(p["W_down"], requires_grad=True)
    X = torch.tensor(p["X"], requires_grad=True)
    tok = torch.as_tensor(r.token, dtype=torch.long)
    ex = torch.as_tensor(r.expert, dtype=torch.long)
    xs = X[tok]
    a = torch.einsum("pih,ph->pi", Wg[ex], xs)
    b = torch.einsum("pih,ph->pi", Wu[ex], xs)
    y = torch.einsum("phi,pi->ph", Wd[ex], torch.nn.functional.silu(a) * b)
    y = torch.tensor(r.weight, dtype=torch.float64)[:, None] * y
    (torch.tensor(p["G"])[tok] * y).sum().backward()
    ref = O.swiglu_reference(p)
    for e in range(r.E):
        assert _rel(ref["dW_down"][e], Wd.grad[e].numpy()) < 1e-12
        assert _rel(ref["dW_gate"][e], Wg.grad[e].numpy()) < 1e-12
        assert _rel(ref["dW_up"][e], Wu.grad[e].numpy()) < 1e-12
    assert _rel(ref["dX"], X.grad.numpy()) < 1e-12


def test_silu_derivative_matches_autograd():
    a = torch.linspace(-12, 12, 2001, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.silu(a).sum().backward()
    an = a.detach().numpy()
    np.testing.assert_allclose(O.dsilu(an), a.grad.numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(O.silu(an), torch.nn.functional.silu(a).detach().numpy(),
                               rtol=1e-13, atol=1e-300)


# ------------------------------------------------- generator determinism

def test_generator_is_deterministic():
    a = synth.make_config(1)
    b = synth.make_config(1)
    for k in ("expert", "token", "weight", "counts"):
        assert np.array_equal(getattr(a["routing"], k), getattr(b["routing"], k))
    for k in ("X", "G", "W"):
        assert torch.equal(a[k], b[k])
    assert np.array_equal(a["quota"], b["quota"])


def test_generator_config_shapes():
    stats = {}
    for i in range(1, 6):
        spec = synth.CONFIGS[i]
        r = synth.make_routing(spec["T"], spec["E"], spec["k"], spec["zipf"], "cfg", i,
                               local=spec.get("local"))
        assert np.all(np.diff(r.token) >= 0)
        assert r.expert.min() >= 0 and r.expert.max() < r.E
        q = synth._quotas(i, r, None)
        assert all((v >= 0).all() for v in q.values())
        stats[i] = (r.N, r.E)
    assert stats[1] == (512, 8) and stats[2] == (32768, 128) and stats[3] == (131072, 128)
    assert stats[4][1] == 32 and stats[5] == (524288, 128)


def test_swiglu_pair_dx_and_given_kept_sets():
    """swiglu_pair_dx equals the per-pair autograd x-gradients through the gate
    and up paths; re-running on given kept sets reproduces the selection run."""
    p = _swiglu_problem(seed=41, quotas=(lambda c: (3 * c) // 4, lambda c: c // 3,
                                         lambda c: c // 2))
    r = p["routing"]
    terms = _swiglu_pair_terms(p)
    ref = O.swiglu_reference(p)
    for e in range(r.E):
        kd = ref["K_down"][e]
        if not kd.size:
            continue
        ing = np.isin(kd, ref["K_gate"][e])
        inu = np.isin(kd, ref["K_up"][e])
        got = O.swiglu_pair_dx(p, kd, ing, inu)
        want = np.stack([terms[q]["xg"] * g + terms[q]["xu"] * u
                         for q, g, u in zip(kd, ing, inu)])
        assert _rel(got, want) < 1e-12
    again = O.swiglu_reference(p, kept={"down": ref["K_down"], "gate": ref["K_gate"],
                                        "up": ref["K_up"]})
    for e in range(r.E):
        for k in ("dW_down", "dW_gate", "dW_up"):
            assert np.array_equal(again[k][e], ref[k][e])
    assert np.array_equal(again["dX"], ref["dX"])


# ------------------------------------------------------------- threshold

def _bruteforce_threshold(score, expert, quota, e):
    """The M_e-th largest score of expert e by a Python sort (None when the
    selection keeps nothing or everything, so there is nothing to decide)."""
    c = sorted((float(score[q]) for q in range(len(score)) if expert[q] == e), reverse=True)
    m = min(int(quota[e]), len(c))
    return None if m in (0, len(c)) else c[m - 1]


def test_threshold_hand_cases():
    # one expert, scores 9 7 4 2 (pair order scrambled), quota 2: the second
    # largest (7) decides, not the third (4) nor the largest (9)
    score = np.array([4.0, 9.0, 2.0, 7.0])
    kept = O.select_top_quota(np.zeros(4, np.int32), score, np.array([2]), 1)[0]
    assert kept.tolist() == [1, 3]
    assert O.threshold(score, kept, 4) == 7.0
    # nothing kept, everything kept: no threshold
    assert O.threshold(score, np.zeros(0, np.int64), 4) is None
    assert O.threshold(score, np.arange(4), 4) is None
    # a single kept pair among several: its own score
    assert O.threshold(score, np.array([1]), 4) == 9.0
    # ties straddling the boundary: scores 5 3 3 3 1, quota 2 keeps 5 and the
    # lowest-index 3; the threshold is 3, equal to the dropped tied pairs
    score = np.array([5.0, 3.0, 3.0, 3.0, 1.0])
    kept = O.select_top_quota(np.zeros(5, np.int32), score, np.array([2]), 1)[0]
    assert kept.tolist() == [0, 1]
    assert O.threshold(score, kept, 5) == 3.0


def test_threshold_against_sorted_scores():
    rng = np.random.default_rng(21)
    for trial in range(20):
        N, E = int(rng.integers(1, 200)), int(rng.integers(1, 6))
        expert = rng.integers(0, E, N).astype(np.int32)
        # few distinct values on odd trials: ties at the boundary
        score = (rng.integers(0, 5, N) if trial % 2 else rng.random(N)).astype(np.float64)
        quota = rng.integers(0, 60, E)
        kept = O.select_top_quota(expert, score, quota, E)
        counts = np.bincount(expert, minlength=E)
        for e in range(E):
            assert O.threshold(score, kept[e], int(counts[e])) == \
                _bruteforce_threshold(score, expert, quota, e)
