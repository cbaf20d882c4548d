"""Benchmark of the LRM-pruned MoE expert backward on one MI355X.

One step = one pass of the whole hot path over one layer call of synthetic
input already resident in HBM: LRM score -> per-expert top-quota select ->
compaction -> grouped GEMM (dW, dX rows) -> unpermute to token layout (and,
for SwiGLU workloads, the chained down -> gate/up stages).

Prints ONE JSON line.  `value` is kept pairs per second of the fused call.
The `roofline` block covers the dominant kernel (the grouped GEMM), timed with
HIP events on the stream it runs on; the `cpu_baseline` block times the fp64
CPU oracle on the host cores.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "kept pairs/s + grouped-GEMM TFLOP/s (% MFMA peak), score/compact GB/s"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return ap.parse_args()


# ------------------------------------------------------------------ LINEAR
class LinearBench:
    """Buffers and per-step calls of a LINEAR workload (all on one stream)."""

    def __init__(self, L, p, dev):
        self.L, self.p = L, p
        r = p["routing"]
        self.r = r
        self.pairs = L.Pairs.from_routing(r, dev)
        self.X, self.G, self.W = (p[k] for k in ("X", "G", "W"))
        self.d_in, self.d_out = p["d_in"], p["d_out"]
        self.quota = np.ascontiguousarray(p["quota"], dtype=np.int32)
        self.Mcap = L.lrm_max_kept(r.N, self.quota)
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        dt = self.X.dtype
        self.score = torch.empty(r.N, **f32)
        self.pos = torch.empty(r.N, **i32)
        self.kept = torch.empty(r.N, **i32)
        self.offsets = torch.empty(r.E + 1, **i32)
        self.Xp = torch.empty(self.Mcap, self.d_in, dtype=dt, device=dev)
        self.Gp = torch.empty(self.Mcap, self.d_out, dtype=dt, device=dev)
        self.dW = torch.empty(r.E, self.d_out, self.d_in, **f32)
        self.dXp = torch.empty(self.Mcap, self.d_in, **f32)
        self.dX = torch.empty(r.T, self.d_in, **f32)
        u8 = dict(dtype=torch.uint8, device=dev)
        lib = L._lib
        import ctypes as C
        self.ws_score = torch.empty(lib.lrm_score_workspace_size(C.byref(self.pairs.c)), **u8)
        self.ws_sel = torch.empty(lib.lrm_select_workspace_size(C.byref(self.pairs.c)), **u8)
        self.ws_gemm = torch.empty(max(lib.lrm_grouped_bwd_workspace_size(r.E), 256), **u8)
        self.ws_unp = torch.empty(lib.lrm_unpermute_workspace_size(C.byref(self.pairs.c)), **u8)
        self.mx = L.mat(self.X, p["X_rows"])
        self.mg = L.mat(self.G, p["G_rows"])
        # fused-call problem (pruned and unpruned)
        self.pb = L.linear_problem(self.pairs, self.X, p["X_rows"], self.G, p["G_rows"], self.W,
                                   self.quota)
        self.pb_full = L.linear_problem(self.pairs, self.X, p["X_rows"], self.G, p["G_rows"],
                                        self.W, None, L.LRM_KEEP_ALL)
        self.ws_fused = torch.empty(L.lrm_workspace_size(self.pb), **u8)
        self.ws_full = torch.empty(L.lrm_workspace_size(self.pb_full), **u8)
        self.out = dict(dW=self.dW, dX=self.dX, pos=self.pos, offsets=self.offsets)
        self.names = ["score", "select", "compact", "grouped_gemm", "unpermute"]

    def step_parts(self, ev=None):
        L = self.L
        if ev: ev[0].record()
        L.lrm_score(self.pairs, self.mx, self.mg, self.score, ws=self.ws_score)
        if ev: ev[1].record()
        L.lrm_select(self.pairs, self.score, self.quota, self.pos, self.offsets, self.kept,
                     ws=self.ws_sel)
        if ev: ev[2].record()
        L.lrm_compact(self.pairs, self.kept, self.offsets, self.Mcap, self.mx, self.mg, self.Xp,
                      self.Gp)
        if ev: ev[3].record()
        L.lrm_grouped_bwd(self.r.E, self.offsets, self.Mcap, self.Gp, self.Xp, self.W, self.d_in,
                          self.d_out, self.dW, self.dXp, ws=self.ws_gemm)
        if ev: ev[4].record()
        L.lrm_unpermute(self.pairs, self.pos, self.dXp, self.d_in, self.p["X_rows"], self.dX,
                        ws=self.ws_unp)
        if ev: ev[5].record()

    def step_fused(self):
        self.L.lrm_expert_backward(self.pb, self.out, ws=self.ws_fused)

    def step_full(self):
        self.L.lrm_expert_backward(self.pb_full, self.out, ws=self.ws_full)

    def kept_rows(self) -> int:
        torch.cuda.synchronize()
        return int(self.offsets[-1].item())

    def work(self, M, active):
        """Algorithmic bytes / flops of each step (what the method must move)."""
        r, p = self.r, self.p
        b = self.X.element_size()
        xr = r.T if p["X_rows"] == "token" else r.N
        gr = r.T if p["G_rows"] == "token" else r.N
        di, do = self.d_in, self.d_out
        return {
            "score": dict(bytes=(xr * di + gr * do) * b + r.N * (4 + 4 + 4)),
            "select": dict(bytes=r.N * (4 + 4) + M * 4),
            "compact": dict(bytes=2 * M * (di + do) * b),
            "grouped_gemm": dict(bytes=r.E * do * di * 4 + active * do * di * b
                                 + M * (di + do) * b + M * di * 4,
                                 flops=4.0 * M * di * do),
            "unpermute": dict(bytes=M * di * 4 + r.T * di * 4),
        }


def time_loop(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_parts(B, steps, warmup):
    for _ in range(warmup):
        B.step_parts()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(B.names) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        B.step_parts(evs[k])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    per = {n: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
           for i, n in enumerate(B.names)}
    return wall, per


def cpu_baseline(p, M):
    from threadpoolctl import threadpool_info

    from oracle import lrm_oracle as O
    host = dict(p, **{k: p[k].cpu() for k in ("X", "G", "W")})
    t0 = time.perf_counter()
    ref = O.linear_reference(host)
    dt = time.perf_counter() - t0
    assert int(ref["offsets"][-1]) == M
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": M / dt, "unit": "kept pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole workload, one pass (score, select, pack, dW, dX) in fp64 NumPy; "
                      f"{dt:.1f} s on {len(os.sched_getaffinity(0))} host cores"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": a.gpus}), flush=True)
        log("bench.py: only --gpus 1 is supported (single-GPU share of the experts)")
        sys.exit(2)
    from pruned_expert_backward_lrm_amd import lrm as L
    from pruned_expert_backward_lrm_amd import synth
    dev = "cuda"
    torch.cuda.set_device(0)
    log(f"bench: generating config {a.config}")
    p = synth.make_config(a.config, device=dev)
    if p["kind"] != "linear":
        raise SystemExit("bench.py: SwiGLU workloads are timed by --config 3..5 in a later build")
    B = LinearBench(L, p, dev)
    r = p["routing"]
    log("bench: timing step-wise path")
    wall_parts, per = time_parts(B, a.steps, a.warmup)
    M = B.kept_rows()
    active = int(np.count_nonzero(np.minimum(p["quota"], r.counts)))
    log("bench: timing fused call")
    ms_fused = time_loop(B.step_fused, a.steps, a.warmup) * 1e3
    log("bench: timing unpruned baseline")
    ms_full = time_loop(B.step_full, a.steps, a.warmup) * 1e3
    work = B.work(M, active)
    g = work["grouped_gemm"]
    t_g = per["grouped_gemm"] * 1e-3
    ai = g["flops"] / g["bytes"]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    gbs = g["bytes"] / t_g / 1e9
    tflops = g["flops"] / t_g / 1e12
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None}
    steps_gbs = {n: round(work[n]["bytes"] / (per[n] * 1e-3) / 1e9, 1) for n in B.names}
    spec = synth.CONFIGS[a.config]
    line = {
        "metric": METRIC,
        "value": round(M / (ms_fused * 1e-3), 1),
        "unit": "kept pairs/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_fused, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{spec['name']}: T={r.T} d_in={p['d_in']} d_out={p['d_out']} "
                               f"E={r.E} top-{r.k} zipf={spec['zipf']} quota=floor(0.6*min(n_e,"
                               f"1.25*mean))",
                   "pairs": r.N, "kept_pairs": M, "active_experts": active},
        "roofline": roof,
        "grouped_gemm": {"ms": round(per["grouped_gemm"], 4), "tflops": round(tflops, 2),
                         "pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                         "gbs": round(gbs, 1), "flops": g["flops"], "bytes": g["bytes"],
                         "arith_intensity": round(ai, 1)},
        "steps_ms": {n: round(v, 4) for n, v in per.items()},
        "steps_gbs": steps_gbs,
        "score_compact_gbs": round((work["score"]["bytes"] + work["compact"]["bytes"])
                                   / ((per["score"] + per["compact"]) * 1e-3) / 1e9, 1),
        "stepwise_ms_per_step": round(wall_parts * 1e3, 4),
        "unpruned_ms_per_step": round(ms_full, 4),
        "kept_fraction": round(M / r.N, 4),
        "pruned_over_unpruned_time": round(ms_fused / ms_full, 4),
    }
    if not a.no_cpu:
        log("bench: timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(p, M)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
