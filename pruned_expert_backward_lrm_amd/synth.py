"""Seeded synthetic workloads for the pruned (LRM) MoE expert backward.

This module only draws inputs: routing (token -> expert pairs with routing
weights), the dense tensors a layer call hands to the backward (saved
projection inputs, incoming gradients, expert weights, saved gate/up
pre-activations) and the per-expert quotas a controller would fix for the
call.  It holds none of the method's arithmetic (no scores, no selection, no
gradients), so both the HIP path and the CPU oracle can be fed from it.

Shapes follow the two models the LRMoE pages train (Qwen3-30B-A3B and
GLM4.5-106B-A12B); the data itself is synthetic.  Conventions:

* pairs are token-major: pair ``p`` belongs to token ``token[p]`` and the
  ``k`` pairs of a token appear in router order (descending logit);
* routing weights are the softmax over a token's ``k`` selected logits;
* "Zipf(s) popularity bias" adds ``-s * ln(rank_e)`` to expert ``e``'s logit,
  with the ranks a seeded permutation of ``1..E``;
* ``N(0, sigma)`` means standard deviation ``sigma``;
* bf16 tensors are fp32 normal draws rounded to nearest-even.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

BASE_SEED = 1234


def _seed(*parts: object) -> int:
    h = hashlib.sha256(repr((BASE_SEED,) + parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal(shape, std, dtype, device, *seed_parts) -> torch.Tensor:
    """Seeded N(0, std) tensor (std is a standard deviation)."""
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*seed_parts))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


@dataclass
class Routing:
    T: int
    E: int            # experts resident (local ids 0..E-1)
    k: int
    expert: np.ndarray  # int32 [N]
    token: np.ndarray   # int32 [N], non-decreasing
    weight: np.ndarray  # float32 [N]
    counts: np.ndarray  # int64 [E], candidates per resident expert
    info: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return int(self.expert.shape[0])


def make_routing(T: int, E: int, k: int, zipf_s: float, *seed_parts,
                 local: tuple[int, int] | None = None) -> Routing:
    """Top-k softmax routing over N(0,1) logits with a Zipf popularity bias.

    ``local=(ranks, which)`` keeps only the pairs whose expert lies in one of
    ``ranks`` contiguous expert blocks: ``which='busiest'`` picks the block
    with the most pairs (the straggler of a synchronous expert-parallel step).
    """
    rng = np.random.default_rng(_seed("routing", *seed_parts))
    logits = rng.standard_normal((T, E), dtype=np.float32).astype(np.float64)
    if zipf_s > 0:
        ranks = rng.permutation(E) + 1
        logits += -zipf_s * np.log(ranks.astype(np.float64))[None, :]
    # top-k per token, in descending logit order (ties broken by expert id)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(logits, order, axis=1)
    top = top - top.max(axis=1, keepdims=True)
    ew = np.exp(top)
    w = ew / ew.sum(axis=1, keepdims=True)
    token = np.repeat(np.arange(T, dtype=np.int32), k)
    expert = order.reshape(-1).astype(np.int32)
    weight = w.reshape(-1).astype(np.float32)
    info = {"E_routed": E}
    E_res = E
    if local is not None:
        nranks, which = local
        per = E // nranks
        blk = expert // per
        loads = np.bincount(blk, minlength=nranks)
        r = int(np.argmax(loads)) if which == "busiest" else int(which)
        keep = blk == r
        token, expert, weight = token[keep], expert[keep] - r * per, weight[keep]
        E_res = per
        info.update({"ep_ranks": nranks, "local_rank": r, "rank_loads": loads.tolist()})
    counts = np.bincount(expert, minlength=E_res).astype(np.int64)
    return Routing(T, E_res, k, expert.astype(np.int32), token.astype(np.int32),
                   weight, counts, info)


# ---------------------------------------------------------------- quota rules
# A controller fixes one integer quota per expert for the whole layer call.
# The rules below stand in for it; all integer arithmetic on the counts.

def quota_half(counts):
    return (counts // 2).astype(np.int32)


def quota_ratio(counts, num, den):
    return (counts * num // den).astype(np.int32)


def quota_capped(counts, N, E):
    """floor(0.6 * min(n_e, 1.25 * N/E)) computed exactly in integers."""
    cap_num, cap_den = 5 * N, 4 * E              # 1.25 * N / E = cap_num / cap_den
    m = np.minimum(counts * cap_den, cap_num)    # min(n_e, cap) * cap_den
    return (3 * m // (5 * cap_den)).astype(np.int32)


def quota_stress(counts, N, E):
    """Kept fraction 1.0 up to the mean load, 0.1 beyond ten times the mean."""
    mean = N // E
    return np.minimum(counts, np.maximum(counts // 10, mean)).astype(np.int32)


# -------------------------------------------------------------- the workloads

CONFIGS = {
    1: dict(name="tiny-linear-fp32", kind="linear", T=256, d_in=64, d_out=128, E=8, k=2,
            zipf=0.0, dtype="f32", g_std=1e-2),
    2: dict(name="qwen3-30b-a3b-linear", kind="linear", T=4096, d_in=2048, d_out=768, E=128,
            k=8, zipf=1.1, dtype="bf16", g_std=1e-3),
    3: dict(name="qwen3-30b-a3b-swiglu", kind="swiglu", T=16384, H=2048, I=768, E=128, k=8,
            zipf=1.2, dtype="bf16", g_std=1e-3),
    4: dict(name="glm4.5-106b-a12b-swiglu-local32", kind="swiglu", T=16384, H=4096, I=1408,
            E=128, k=8, zipf=1.2, dtype="bf16", g_std=1e-3, local=(4, "busiest")),
    5: dict(name="heavy-skew-swiglu", kind="swiglu", T=65536, H=4096, I=1408, E=128, k=8,
            zipf=1.6, dtype="bf16", g_std=1e-3),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _quotas(cfg_id: int, r: Routing, variant: str | None) -> dict:
    c, N, E = r.counts, r.N, r.E
    if cfg_id == 1:
        return {"quota": quota_half(c)}
    if cfg_id == 2:
        return {"quota": quota_capped(c, N, E)}
    if cfg_id == 3:
        qd = quota_half(c)
        if variant == "3b":
            # second selection: gate/up keep half of what the down stage kept
            kd = np.minimum(qd, c)
            qg = (kd // 2).astype(np.int32)
            return {"quota_down": qd, "quota_gate": qg, "quota_up": qg.copy()}
        return {"quota_down": qd, "quota_gate": qd.copy(), "quota_up": qd.copy()}
    if cfg_id == 4:
        q = quota_ratio(c, 3, 5)
        return {"quota_down": q, "quota_gate": q.copy(), "quota_up": q.copy()}
    if cfg_id == 5:
        q = quota_stress(c, N, E)
        return {"quota_down": q, "quota_gate": q.copy(), "quota_up": q.copy()}
    raise ValueError(cfg_id)


def make_config(cfg_id: int, device: str = "cpu", variant: str | None = None) -> dict:
    """Materialise one of the five workloads.  Dense tensors live on ``device``."""
    spec = CONFIGS[cfg_id]
    r = make_routing(spec["T"], spec["E"], spec["k"], spec["zipf"], "cfg", cfg_id,
                     local=spec.get("local"))
    dt = torch_dtype(spec["dtype"])
    out = dict(cfg=cfg_id, name=spec["name"], kind=spec["kind"], dtype=spec["dtype"],
               routing=r, T=r.T, N=r.N, E=r.E, k=r.k)
    out.update(_quotas(cfg_id, r, variant))
    if spec["kind"] == "linear":
        d_in, d_out = spec["d_in"], spec["d_out"]
        out.update(d_in=d_in, d_out=d_out, X_rows="token", G_rows="pair",
                   X=normal((r.T, d_in), 1.0, dt, device, "cfg", cfg_id, "X"),
                   G=normal((r.N, d_out), spec["g_std"], dt, device, "cfg", cfg_id, "G"),
                   W=normal((r.E, d_out, d_in), 0.02, dt, device, "cfg", cfg_id, "W"))
    else:
        H, I = spec["H"], spec["I"]
        out.update(H=H, I=I,
                   X=normal((r.T, H), 1.0, dt, device, "cfg", cfg_id, "X"),
                   G=normal((r.T, H), spec["g_std"], dt, device, "cfg", cfg_id, "G"),
                   A=normal((r.N, I), 1.0, dt, device, "cfg", cfg_id, "A"),
                   B=normal((r.N, I), 1.0, dt, device, "cfg", cfg_id, "B"),
                   W_gate=normal((r.E, I, H), 0.02, dt, device, "cfg", cfg_id, "Wg"),
                   W_up=normal((r.E, I, H), 0.02, dt, device, "cfg", cfg_id, "Wu"),
                   W_down=normal((r.E, H, I), 0.02, dt, device, "cfg", cfg_id, "Wd"))
    return out


def make_linear(T, E, k, d_in, d_out, *, dtype="f32", x_rows="token", g_rows="pair",
                zipf=0.0, quota=None, device="cpu", seed=0, g_std=1e-2,
                local=None) -> dict:
    """A LINEAR problem of arbitrary shape (for edge-case and parity tests).

    ``quota`` is an int array, a callable on the counts, or None (half).
    """
    r = make_routing(T, E, k, zipf, "lin", seed, T, E, k, local=local)
    dt = torch_dtype(dtype)
    xr = r.T if x_rows == "token" else r.N
    gr = r.T if g_rows == "token" else r.N
    if quota is None:
        q = quota_half(r.counts)
    elif callable(quota):
        q = np.asarray(quota(r.counts), dtype=np.int32)
    else:
        q = np.asarray(quota, dtype=np.int32)
    return dict(kind="linear", dtype=dtype, routing=r, T=r.T, N=r.N, E=r.E, k=k,
                d_in=d_in, d_out=d_out, X_rows=x_rows, G_rows=g_rows, quota=q,
                X=normal((xr, d_in), 1.0, dt, device, "lin", seed, "X"),
                G=normal((gr, d_out), g_std, dt, device, "lin", seed, "G"),
                W=normal((r.E, d_out, d_in), 0.02, dt, device, "lin", seed, "W"))


def make_swiglu(T, E, k, H, I, *, dtype="bf16", zipf=0.0, quotas=None, device="cpu",
                seed=0, g_std=1e-3, local=None) -> dict:
    """A SwiGLU problem of arbitrary shape.  ``quotas`` = (down, gate, up)."""
    r = make_routing(T, E, k, zipf, "glu", seed, T, E, k, local=local)
    dt = torch_dtype(dtype)
    if quotas is None:
        qd = quota_half(r.counts)
        quotas = (qd, qd.copy(), qd.copy())
    qd, qg, qu = (np.asarray(q(r.counts) if callable(q) else q, dtype=np.int32) for q in quotas)
    return dict(kind="swiglu", dtype=dtype, routing=r, T=r.T, N=r.N, E=r.E, k=k, H=H, I=I,
                quota_down=qd, quota_gate=qg, quota_up=qu,
                X=normal((r.T, H), 1.0, dt, device, "glu", seed, "X"),
                G=normal((r.T, H), g_std, dt, device, "glu", seed, "G"),
                A=normal((r.N, I), 1.0, dt, device, "glu", seed, "A"),
                B=normal((r.N, I), 1.0, dt, device, "glu", seed, "B"),
                W_gate=normal((r.E, I, H), 0.02, dt, device, "glu", seed, "Wg"),
                W_up=normal((r.E, I, H), 0.02, dt, device, "glu", seed, "Wu"),
                W_down=normal((r.E, H, I), 0.02, dt, device, "glu", seed, "Wd"))


def describe(cfg: dict) -> dict:
    """Load statistics of a workload (counts only; no method arithmetic)."""
    r: Routing = cfg["routing"]
    c = r.counts
    return {"T": r.T, "N": r.N, "E": r.E, "k": r.k, "max_count": int(c.max()) if c.size else 0,
            "mean_count": float(c.mean()) if c.size else 0.0,
            "zero_count_experts": int((c == 0).sum()), **r.info}
