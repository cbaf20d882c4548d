"""Benchmark of the LRM-pruned MoE expert backward on one MI355X.

One step = one pass of the whole hot path over one layer call of synthetic
input already resident in HBM, through the fused C-ABI call: LRM score ->
per-expert top-quota select -> compaction -> grouped GEMM (dW, dX rows) ->
unpermute to token layout; SwiGLU workloads chain down -> gate/up stages.

Prints ONE JSON line.  `value` is kept pairs per second of the fused call
(for SwiGLU, pairs kept by the down stage), over K plain fused calls.  Stage
times come from a second pass of K calls in which the library records HIP
events on its launch stream at stage boundaries; the
`roofline` block covers the dominant kernel: for a linear layer the longer
of the two grouped-GEMM launches (dW or dX), timed alone with HIP events on
the packed operands of the same call; its `traffic` comes from the committed
counter runs when they match the kernel source; the `cpu_baseline` block
times the fp64 CPU oracle on the host cores.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu] [--full]

`--redistribute` instead prints one JSON line on the redistribution of the
kept pairs over G=8 GPUs (each expert owned by one, the 16 most loaded
replicated on all): the host solver's time and the device layout's time on
the workload's real selection, and the optimal peak against fixed ownership.

`--controller` instead prints one JSON line comparing the fused call under
the workload's own quotas with the same pair budget spent by the quota
controller (water-filling caps, lrm_quota_waterfill).

`--sweep` instead prints one JSON line of the keep-ratio sweep: the fused call
with every quota at floor(r * n_e) for r in 0.1, 0.25, 0.5, 0.75, 1.0 (all
projections alike), and the unpruned call, on the chosen workload.

The HBM-traffic record the `roofline.traffic` field reads is written on any
host, without a GPU, from two profiler passes over `--copy-probe` runs:

    python bench.py --record-traffic FETCH_DIR WRITE_DIR [--config 2]
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
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--variant", default=None, help="3b: a real gate/up second selection")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--full", action="store_true",
                    help="also time the unpruned (keep-all) call: its GEMM launches run other "
                         "shapes, so it is off by default to keep the kernel statistics of a "
                         "profiled bench run those of the pruned call")
    ap.add_argument("--no-full", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 512 MiB device copy (a known-size kernel that "
                         "calibrates the HBM byte counters of a profiler pass)")
    ap.add_argument("--h-table", action="store_true",
                    help="SwiGLU: pass the per-pair |silu(a) b|^2 a forward pass would save "
                         "(computed before timing), so the down score reads no A/B rows")
    ap.add_argument("--dw-bf16", action="store_true",
                    help="weight gradients stored as bf16 (LRM_DW_BF16) instead of fp32")
    ap.add_argument("--controller", action="store_true",
                    help="compare the workload's quotas with water-filling quotas of equal budget")
    ap.add_argument("--redistribute", action="store_true",
                    help="time the redistribution onto replicas instead of the bench line")
    ap.add_argument("--sweep", action="store_true",
                    help="keep-ratio sweep (quota = floor(r n_e)) instead of the bench line")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/hbm_traffic.json from the output folders of a "
                         "rocprofv3 --pmc FETCH_SIZE and a --pmc WRITE_SIZE pass over "
                         "`bench.py --no-cpu --copy-probe` (no GPU needed)")
    return ap.parse_args()


COPY_KIB = 512 * 1024  # bytes moved each way by one copy of copy_probe, in KiB
TRAFFIC_PATH = os.path.join(ROOT, "profiles", "hbm_traffic.json")
GEMM_SRC = os.path.join(ROOT, "pruned_expert_backward_lrm_amd", "csrc", "k_gemm.hip")


def normalized_source(text):
    """C++ source without comments and whitespace: edits of comments or layout
    do not change what the counters were taken on."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "".join(text.split())


def gemm_source_sha():
    import hashlib
    with open(GEMM_SRC, encoding="utf-8") as f:
        return hashlib.sha256(normalized_source(f.read()).encode()).hexdigest()


def workload_name(spec, T, E, k, shape, variant=None):
    return f"{spec['name']}{'-' + variant if variant else ''}: {shape} E={E} top-{k} zipf={spec['zipf']}"


def gemm_work(E, Me, d_in, d_out, b):
    """Algorithmic bytes and flops of the two grouped-GEMM launches of a
    linear layer call with kept counts Me: the dW launch writes every
    expert's fp32 dW and reads the packed rows once; the dX launch reads W of
    the active experts and the packed G rows, and writes the fp32 dX rows."""
    M, act = int(np.sum(Me)), int(np.count_nonzero(Me))
    return {
        "dW": dict(bytes=E * d_out * d_in * 4 + M * (d_in + d_out) * b, flops=2.0 * M * d_in * d_out),
        "dX": dict(bytes=act * d_out * d_in * b + M * d_out * b + M * d_in * 4,
                   flops=2.0 * M * d_in * d_out),
    }


def record_traffic(fetch_dir, write_dir, cfg):
    """profiles/hbm_traffic.json from two counter passes: per GEMM launch, the
    average FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the same
    counter reads for the three 512 MiB copies of --copy-probe."""
    import csv
    import glob

    from pruned_expert_backward_lrm_amd import synth
    spec = synth.CONFIGS[cfg]
    if spec["kind"] != "linear":
        raise SystemExit("--record-traffic covers the linear workloads (one dW and one dX launch)")
    r = synth.make_routing(spec["T"], spec["E"], spec["k"], spec["zipf"], "cfg", cfg,
                           local=spec.get("local"))
    q = synth._quotas(cfg, r, None)["quota"]
    Me = np.minimum(np.maximum(q, 0), r.counts).astype(np.int64)
    b = torch.tensor([], dtype=synth.torch_dtype(spec["dtype"])).element_size()
    work = gemm_work(r.E, Me, spec["d_in"], spec["d_out"], b)
    workload = workload_name(spec, r.T, r.E, r.k,
                             f"T={r.T} d_in={spec['d_in']} d_out={spec['d_out']}")
    per, scale, names = {"dW": {}, "dX": {}}, {}, {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [row for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                                       recursive=True)
                for row in csv.DictReader(open(f)) if row["Counter_Name"] == counter]
        rows.sort(key=lambda row: int(row["Dispatch_Id"]))
        copies = [float(row["Counter_Value"]) for row in rows
                  if row["Kernel_Name"] == "__amd_rocclr_copyBuffer"][:3]
        if len(copies) != 3:
            raise SystemExit(f"{d}: no --copy-probe copies found for {counter}")
        scale[counter] = float(np.mean(copies)) / COPY_KIB
        for kind, tail in (("dW", "false>(lrm::GemmPlan)"), ("dX", "true>(lrm::GemmPlan)")):
            vals = [float(row["Counter_Value"]) for row in rows
                    if "k_gemm_stream<" in row["Kernel_Name"] and row["Kernel_Name"].endswith(tail)]
            if not vals:
                raise SystemExit(f"{d}: no {kind} grouped-GEMM dispatches")
            names[kind] = next(row["Kernel_Name"] for row in rows
                               if "k_gemm_stream<" in row["Kernel_Name"]
                               and row["Kernel_Name"].endswith(tail))
            per[kind][counter] = (float(np.mean(vals)), len(vals))
    sha = gemm_source_sha()
    kernels = []
    for kind in ("dW", "dX"):
        fk, n = per[kind]["FETCH_SIZE"]
        wk, _ = per[kind]["WRITE_SIZE"]
        fb = fk / scale["FETCH_SIZE"] * 1024
        wb = wk / scale["WRITE_SIZE"] * 1024
        alg = work[kind]["bytes"]
        kernels.append({"kernel": f"k_gemm_stream<{kind}>", "profiler_name": names[kind],
                        "workload": workload, "source_sha256": sha, "dispatches": n,
                        "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
                        "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
                        "hbm_bytes": int(round(fb + wb)), "algorithmic_bytes": int(alg),
                        "traffic_over_algorithmic": round((fb + wb) / alg, 3)})
    rec = {
        "note": ("HBM bytes per launch of the grouped-GEMM kernels, from two rocprofv3 --pmc "
                 "passes (FETCH_SIZE, WRITE_SIZE, KiB per dispatch) scaled by what the same "
                 f"counters read for a 512 MiB device copy (FETCH_SIZE reads "
                 f"{scale['FETCH_SIZE']:.4f}, WRITE_SIZE {scale['WRITE_SIZE']:.4f} of the true "
                 "bytes). source_sha256 is the SHA-256 of csrc/k_gemm.hip, comments and "
                 "whitespace removed, that the counters were taken on."),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d " + fetch_dir
            + f" -o run -- python bench.py --config {cfg} --no-cpu --copy-probe --steps 5 --warmup 2",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d " + write_dir
            + f" -o run -- python bench.py --config {cfg} --no-cpu --copy-probe --steps 5 --warmup 2",
            f"python bench.py --config {cfg} --record-traffic {fetch_dir} {write_dir}",
        ],
        "kernels": kernels,
    }
    with open(TRAFFIC_PATH, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def copy_probe(dev):
    """A device-to-device copy of exactly 512 MiB (read 512 MiB, write 512 MiB)."""
    n = 512 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


class Workload:
    """Problem descriptors, outputs and workspaces of one layer call."""

    def __init__(self, L, p, dev, dw_bf16=False, h_table=False):
        self.L, self.p, self.r = L, p, p["routing"]
        self.dwb = dw_bf16
        self.htab = None
        if h_table and p["kind"] != "linear":
            # what a forward pass would save: |silu(a) b|^2 per pair, fp64
            A, B = p["A"], p["B"]
            self.htab = torch.empty(A.shape[0], dtype=torch.float64, device=dev)
            for i in range(0, A.shape[0], 1 << 16):
                a, b = A[i:i + (1 << 16)].float(), B[i:i + (1 << 16)].float()
                h = a * torch.sigmoid(a) * b
                self.htab[i:i + (1 << 16)] = (h * h).sum(dim=1, dtype=torch.float64)
        fl = L.LRM_DW_BF16 if dw_bf16 else 0
        wdt = torch.bfloat16 if dw_bf16 else torch.float32
        r = self.r
        self.pairs = L.Pairs.from_routing(r, dev)
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.kind = p["kind"]
        if self.kind == "linear":
            X, G, W = p["X"], p["G"], p["W"]
            self.pb = L.linear_problem(self.pairs, X, p["X_rows"], G, p["G_rows"], W, p["quota"],
                                       fl)
            self.pb_full = L.linear_problem(self.pairs, X, p["X_rows"], G, p["G_rows"], W, None,
                                            L.LRM_KEEP_ALL | fl)
            rows = r.T if p["X_rows"] == "token" else r.N
            self.out = dict(dW=torch.empty(r.E, p["d_out"], p["d_in"], dtype=wdt, device=dev),
                            dX=torch.empty(rows, p["d_in"], **f32))
            self.stages = ["score", "select", "compact", "grouped_gemm", "unpermute"]
            self.gemm_stages = ["grouped_gemm"]
        else:
            t = [p[k] for k in ("X", "G", "A", "B", "W_gate", "W_up", "W_down")]
            q = (p["quota_down"], p["quota_gate"], p["quota_up"])
            self.pb = L.swiglu_problem(self.pairs, t[0], "token", t[1], "token", *t[2:], *q, fl,
                                       h_sumsq=self.htab)
            self.pb_full = L.swiglu_problem(self.pairs, t[0], "token", t[1], "token", *t[2:],
                                            None, None, None, L.LRM_KEEP_ALL | fl)
            H, I = p["H"], p["I"]
            wd = dict(dtype=wdt, device=dev)
            self.out = dict(dW_gate=torch.empty(r.E, I, H, **wd),
                            dW_up=torch.empty(r.E, I, H, **wd),
                            dW_down=torch.empty(r.E, H, I, **wd), dX=torch.empty(r.T, H, **f32))
            self.stages = ["score_down", "select_down", "compact_down", "gemm_down", "glu_bwd",
                           "select_gate_up", "compact_gate_up", "gemm_gate_up", "unpermute"]
            self.gemm_stages = ["gemm_down", "gemm_gate_up"]
        self.out["offsets"] = torch.empty(r.E + 1, **i32)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws = torch.empty(L.lrm_workspace_size(self.pb), **u8)
        self.ws_full = torch.empty(L.lrm_workspace_size(self.pb_full), **u8)
        self.out_full = dict(self.out)
        self.out_full["offsets"] = torch.empty(r.E + 1, **i32)

    def step(self, events=None):
        if events is None:
            self.L.lrm_expert_backward(self.pb, self.out, ws=self.ws)
        else:
            self.L.lrm_expert_backward_events(self.pb, self.out, events, ws=self.ws)

    def step_full(self):
        self.L.lrm_expert_backward(self.pb_full, self.out_full, ws=self.ws_full)

    def kept(self):
        torch.cuda.synchronize()
        offs = self.out["offsets"].cpu().numpy().astype(np.int64)
        return int(offs[-1]), np.diff(offs)

    def work(self, M, Me):
        """Algorithmic bytes (and flops) of each stage: what the method must
        move, with the packed rows counted once and fp32 outputs."""
        p, r = self.p, self.r
        b = self.p["X"].element_size()
        wb = 2 if self.dwb else 4  # bytes of a stored weight-gradient element
        act = int(np.count_nonzero(Me))
        E, N, T = r.E, r.N, r.T
        if self.kind == "linear":
            di, do = p["d_in"], p["d_out"]
            xr = T if p["X_rows"] == "token" else N
            gr = T if p["G_rows"] == "token" else N
            return {
                "score": dict(bytes=(xr * di + gr * do) * b + N * 12),
                "select": dict(bytes=N * 8 + M * 4),
                "compact": dict(bytes=2 * M * (di + do) * b),
                "grouped_gemm": dict(bytes=E * do * di * wb + act * do * di * b
                                     + M * (di + do) * b + M * di * 4,
                                     flops=4.0 * M * di * do),
                "unpermute": dict(bytes=M * di * 4 + T * di * 4),
            }
        H, I = p["H"], p["I"]
        return {
            "score_down": dict(bytes=T * H * b + (N * 8 if self.htab is not None else 2 * N * I * b)
                               + N * 12),
            "select_down": dict(bytes=N * 8 + M * 4),
            "compact_down": dict(bytes=2 * M * H * b + 3 * M * I * b),
            "gemm_down": dict(bytes=act * H * I * b + E * H * I * wb + M * (H + I) * b
                              + M * I * 4, flops=4.0 * M * H * I),
            "glu_bwd": dict(bytes=T * H * b + M * I * 4 + 4 * M * I * b),
            "select_gate_up": dict(bytes=2 * (M * 8)),
            "compact_gate_up": dict(bytes=2 * M * H * b),
            "gemm_gate_up": dict(bytes=2 * act * I * H * b + 2 * E * I * H * wb
                                 + M * (2 * I + H) * b + M * H * 4, flops=8.0 * M * H * I),
            "unpermute": dict(bytes=M * H * 4 + T * H * 4),
        }


def time_fused(W, steps, warmup):
    """Wall time per step of the plain fused call (the timed region holds the
    steps only), then the per-stage split from a second pass of the same
    steps with HIP events recorded at the stage boundaries (the events cost a
    little GPU time of their own, so they stay out of the first pass)."""
    wall = time_loop(W.step, steps, warmup)
    n = len(W.stages) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(steps)]
    for row in evs:  # materialise the event handles
        for ev in row:
            ev.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        W.step(evs[k])
    torch.cuda.synchronize()
    wall_ev = (time.perf_counter() - t0) / steps
    per = {name: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
           for i, name in enumerate(W.stages)}
    return wall, per, wall_ev


def gemm_kernels(W, steps, warmup):
    """Times the two grouped-GEMM launches of a linear layer call on their
    own, on the same packed operands the fused call builds: the dW kernel
    (dW_e = Gp_e^T Xp_e) and the dX kernel (dXp_e = Gp_e W_e).  HIP events on
    the launch stream around `steps` launches each.  Returns, per kernel, the
    average launch duration and its algorithmic bytes and flops."""
    L, p, r = W.L, W.p, W.r
    dev = W.out["dW"].device
    i32 = dict(dtype=torch.int32, device=dev)
    X, G = L.mat(p["X"], p["X_rows"]), L.mat(p["G"], p["G_rows"])
    score = torch.empty(r.N, dtype=torch.float32, device=dev)
    L.lrm_score(W.pairs, X, G, score)
    pos, kept = torch.empty(r.N, **i32), torch.empty(max(r.N, 1), **i32)
    offsets = torch.empty(r.E + 1, **i32)
    L.lrm_select(W.pairs, score, p["quota"], pos, offsets, kept, device=dev)
    M = int(offsets[-1].item())
    di, do = p["d_in"], p["d_out"]
    Xp = torch.empty(max(M, 1), di, dtype=p["X"].dtype, device=dev)
    Gp = torch.empty(max(M, 1), do, dtype=p["G"].dtype, device=dev)
    L.lrm_compact(W.pairs, kept, offsets, M, X, G, Xp, Gp)
    dW = torch.empty(r.E, do, di, dtype=torch.float32, device=dev)
    dXp = torch.empty(max(M, 1), di, dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    Me = np.diff(offsets.cpu().numpy().astype(np.int64))
    work = gemm_work(r.E, Me, di, do, p["X"].element_size())
    runs = {
        "dW": (lambda: L.lrm_grouped_bwd(r.E, offsets, M, Gp, Xp, p["W"], di, do, dW, None, ws=ws),
               work["dW"]),
        "dX": (lambda: L.lrm_grouped_bwd(r.E, offsets, M, Gp, Xp, p["W"], di, do, None, dXp, ws=ws),
               work["dX"]),
    }
    res = {}
    for name, (fn, work) in runs.items():
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = dict(work, ms=e0.elapsed_time(e1) / steps)
    return res


def traffic_of(kernel, workload):
    """HBM bytes per launch from the committed counter runs (profiles/
    hbm_traffic.json), or None when they were taken on another workload or on
    another version of the kernel source."""
    try:
        with open(TRAFFIC_PATH) as f:
            rec = json.load(f)
        sha = gemm_source_sha()
    except (OSError, ValueError):
        return None
    for e in rec.get("kernels", []):
        if e.get("kernel") == kernel and e.get("workload") == workload and e.get("source_sha256") == sha:
            return e.get("hbm_bytes")
    return None


def copy_gbs(dev, reps=10):
    """Measured device-copy bandwidth (read + write bytes of a 512 MiB copy
    per second): the practical ceiling of a streaming kernel on this GPU."""
    n = 512 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def attainable_tflops(ai, peak_tf):
    """min(MFMA peak, arithmetic intensity x HBM peak), in TFLOP/s."""
    return min(peak_tf, ai * PEAK_HBM_GBS / 1000.0)


def keep_sweep(L, synth, p, dev, steps, warmup, cfg):
    """Fused-call time with every quota at floor(r n_e), r in RATIOS, and the
    unpruned (keep-all) call, on one workload."""
    ratios = ((1, 10), (1, 4), (1, 2), (3, 4), (1, 1))
    r = p["routing"]
    W = Workload(L, p, dev)
    points = []
    for num, den in ratios:
        q = ((num * r.counts.astype(np.int64)) // den).astype(np.int32)
        if p["kind"] == "linear":
            pb = L.linear_problem(W.pairs, p["X"], p["X_rows"], p["G"], p["G_rows"], p["W"], q)
        else:
            pb = L.swiglu_problem(W.pairs, p["X"], "token", p["G"], "token", p["A"], p["B"],
                                  p["W_gate"], p["W_up"], p["W_down"], q, q, q)
        ws = torch.empty(L.lrm_workspace_size(pb), dtype=torch.uint8, device=dev)
        fn = lambda: L.lrm_expert_backward(pb, W.out, ws=ws)  # noqa: E731
        t = time_loop(fn, steps, warmup)
        M = int(W.out["offsets"][-1].item())
        points.append({"r": num / den, "kept_pairs": M, "kept_fraction": round(M / r.N, 4),
                       "ms": round(t * 1e3, 4), "kept_pairs_per_s": round(M / t, 1)})
        del pb, ws
    t_full = time_loop(W.step_full, steps, warmup)
    for pt in points:
        pt["time_over_unpruned"] = round(pt["ms"] / (t_full * 1e3), 4)
    spec = synth.CONFIGS[cfg]
    return {"metric": "keep-ratio sweep of the fused call", "config": {"workload": spec["name"],
            "pairs": r.N}, "unit": "ms", "steps": steps, "warmup": warmup,
            "unpruned_ms": round(t_full * 1e3, 4), "points": points}


def controller(L, p, dev, steps, warmup):
    """The fused call under the workload's quotas and under water-filling
    quotas (lrm_quota_waterfill) with the same pair budget: kept pairs, the
    largest per-expert kept count, the host controller's time, ms per call."""
    r = p["routing"]
    W = Workload(L, p, dev)
    key = "quota" if p["kind"] == "linear" else "quota_down"
    own = np.asarray(p[key], np.int64)
    budget = int(np.minimum(own, r.counts).sum())
    t0 = time.perf_counter()
    for _ in range(steps):
        wf = L.lrm_quota_waterfill(r.counts, budget)
    t_ctl = (time.perf_counter() - t0) / steps
    res = {}
    for name, q in (("workload_quotas", own.astype(np.int32)), ("waterfill", wf)):
        if p["kind"] == "linear":
            pb = L.linear_problem(W.pairs, p["X"], p["X_rows"], p["G"], p["G_rows"], p["W"], q)
        else:
            pb = L.swiglu_problem(W.pairs, p["X"], "token", p["G"], "token", p["A"], p["B"],
                                  p["W_gate"], p["W_up"], p["W_down"], q, q, q)
        ws = torch.empty(L.lrm_workspace_size(pb), dtype=torch.uint8, device=dev)
        t = time_loop(lambda: L.lrm_expert_backward(pb, W.out, ws=ws), steps, warmup)
        Me = np.diff(W.out["offsets"].cpu().numpy().astype(np.int64))
        res[name] = {"kept_pairs": int(Me.sum()), "max_expert_kept": int(Me.max()),
                     "ms": round(t * 1e3, 4), "kept_pairs_per_s": round(Me.sum() / t, 1)}
        del pb, ws
    return {"metric": "quota controller (water-filling caps) at the workload's pair budget",
            "budget_pairs": budget, "controller_host_us": round(t_ctl * 1e6, 2),
            "steps": steps, "warmup": warmup, **res}


def redistribution(L, p, dev, steps, warmup, G=8, hot=16):
    """Redistribution of one layer call's kept pairs over G GPUs: the host
    solver (lrm_redistribute) and the device receiver-major layout
    (lrm_receiver_layout, HIP events on its stream)."""
    r = p["routing"]
    W = Workload(L, p, dev)
    W.step()
    offsets = W.out["offsets"]
    Me = np.diff(offsets.cpu().numpy().astype(np.int64))
    Rm = np.zeros((r.E, G), bool)
    Rm[np.arange(r.E), np.arange(r.E) % G] = True
    Rm[np.argsort(-Me, kind="stable")[:hot]] = True
    fixed = int(max(Me[np.arange(r.E) % G == g].sum() for g in range(G)))
    for _ in range(warmup):
        L.lrm_redistribute(Me, Rm)
    t0 = time.perf_counter()
    for _ in range(steps):
        peak, x = L.lrm_redistribute(Me, Rm)
    t_host = (time.perf_counter() - t0) / steps
    xd = torch.as_tensor(x, device=dev)
    M = int(Me.sum())
    ws = None
    for _ in range(warmup):
        *_, ws = L.lrm_receiver_layout(offsets, xd, M, ws=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        L.lrm_receiver_layout(offsets, xd, M, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    if L.lrm_check_device_errors(ws) != 0:
        raise RuntimeError("receiver layout flagged the assignment")
    return {"metric": "redistribution of kept pairs onto replicas", "gpus": G,
            "replicated_experts": hot, "kept_pairs": M, "peak_pairs": peak,
            "fixed_ownership_peak_pairs": fixed, "mean_pairs": round(M / G, 1),
            "solver_host_us": round(t_host * 1e6, 1),
            "layout_device_us": round(e0.elapsed_time(e1) / steps * 1e3, 2),
            "steps": steps, "warmup": warmup}


def time_loop(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def cpu_baseline(p, M, Me):
    from threadpoolctl import threadpool_info

    from oracle import lrm_oracle as O
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    cores = len(os.sched_getaffinity(0))
    if p["kind"] == "linear":
        host = dict(p, **{k: p[k].cpu() for k in ("X", "G", "W")})
        t0 = time.perf_counter()
        ref = O.linear_reference(host)
        dt = time.perf_counter() - t0
        assert int(ref["offsets"][-1]) == M
        return {"value": M / dt, "unit": "kept pairs/s", "cores": int(threads), "kind": "oracle",
                "sample": f"the whole workload, one pass (score, select, pack, dW, dX) in fp64 "
                          f"NumPy; {dt:.1f} s on {cores} host cores"}
    # SwiGLU: all down scores and selections, then the full backward of a
    # sample of experts holding about 5% of the kept rows
    host = dict(p, **{k: p[k].cpu() for k in ("X", "G", "A", "B", "W_gate", "W_up", "W_down")})
    order = np.argsort(Me)
    ex, tot = [], 0
    for e in order[::-1][::7]:
        if tot > 0.05 * M:
            break
        if Me[e] > 0:
            ex.append(int(e))
            tot += int(Me[e])
    t0 = time.perf_counter()
    O.swiglu_reference(host, experts=ex)
    dt = time.perf_counter() - t0
    return {"value": tot / dt, "unit": "kept pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": f"down scores and selections of all {p['routing'].N} pairs, then the full "
                      f"backward of {len(ex)} experts holding {tot} of {M} kept pairs; "
                      f"{dt:.1f} s on {cores} host cores"}


def main():
    a = parse()
    if a.record_traffic:
        record_traffic(a.record_traffic[0], a.record_traffic[1], a.config)
        return
    if a.gpus != 1:
        log("bench.py: this build runs on exactly one GPU (one GPU's share of the experts); "
            "--gpus must be 1")
        sys.exit(2)
    from pruned_expert_backward_lrm_amd import lrm as L
    from pruned_expert_backward_lrm_amd import synth
    dev = "cuda"
    torch.cuda.set_device(0)
    if a.copy_probe:
        copy_probe(dev)
    log(f"bench: generating config {a.config}")
    p = synth.make_config(a.config, device=dev, variant=a.variant)
    if a.controller:
        log("bench: quota controller")
        line = controller(L, p, dev, a.steps, a.warmup)
        line["config"] = {"workload": synth.CONFIGS[a.config]["name"]}
        print(json.dumps(line), flush=True)
        return
    if a.redistribute:
        log("bench: redistribution onto replicas")
        line = redistribution(L, p, dev, a.steps, a.warmup)
        line["config"] = {"workload": synth.CONFIGS[a.config]["name"]}
        print(json.dumps(line), flush=True)
        return
    if a.sweep:
        log("bench: keep-ratio sweep")
        print(json.dumps(keep_sweep(L, synth, p, dev, a.steps, a.warmup, a.config)), flush=True)
        return
    W = Workload(L, p, dev, a.dw_bf16, a.h_table)
    r = p["routing"]
    log("bench: timing the pruned backward")
    wall, per, wall_ev = time_fused(W, a.steps, a.warmup)
    M, Me = W.kept()
    ms_full = None
    if a.full and not a.no_full:
        log("bench: timing the unpruned backward (every pair kept)")
        ms_full = time_loop(W.step_full, a.steps, a.warmup) * 1e3
    work = W.work(M, Me)
    flops = sum(work[s]["flops"] for s in W.gemm_stages)
    gbytes = sum(work[s]["bytes"] for s in W.gemm_stages)
    t_g = sum(per[s] for s in W.gemm_stages) * 1e-3
    ai = flops / gbytes
    peak_tf = PEAK_TFLOPS[p["dtype"]]
    ridge = peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
    gbs = gbytes / t_g / 1e9
    tflops = flops / t_g / 1e12
    spec = synth.CONFIGS[a.config]
    if p["kind"] == "linear":
        shape = f"T={r.T} d_in={p['d_in']} d_out={p['d_out']}"
    else:
        shape = f"T={r.T} H={p['H']} I={p['I']}"
    workload = workload_name(spec, r.T, r.E, r.k, shape, a.variant)
    kernels = None
    if p["kind"] == "linear" and not a.dw_bf16:
        # the dominant kernel: the longer of the two GEMM launches, timed alone
        log("bench: timing the grouped-GEMM kernels alone")
        kernels = gemm_kernels(W, a.steps, a.warmup)
        name = max(kernels, key=lambda k: kernels[k]["ms"])
        kd = kernels[name]
        # bf16 runs the two stream kernels; fp32 one tiled FMA kernel over either tile kind
        kname = (f"k_gemm_stream<{name}>" if p["dtype"] == "bf16"
                 else f"k_grouped_gemm_f32 ({name} tiles)")
        k_ai, k_t = kd["flops"] / kd["bytes"], kd["ms"] * 1e-3
        k_gbs, k_tf = kd["bytes"] / k_t / 1e9, kd["flops"] / k_t / 1e12
        traffic = traffic_of(kname, workload)
    else:
        # SwiGLU: the GEMM stages as a whole (several launches)
        kname, k_ai, k_gbs, k_tf, traffic = "gemm stages", ai, gbs, tflops, None
    if k_ai < ridge:
        roof = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(k_gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(k_tf, 2), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(k_tf / peak_tf, 4), "traffic": traffic}
    roof["kernel"] = kname
    mem_stages = [s for s in W.stages if s not in W.gemm_stages]
    log("bench: measuring device-copy bandwidth")
    cgbs = copy_gbs(dev)
    sc = [s for s in W.stages if s.startswith("score") or s.startswith("compact")]
    line = {
        "metric": METRIC,
        "value": round(M / wall, 1),
        "unit": "kept pairs/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "ms_per_step_with_stage_events": round(wall_ev * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p["dtype"],
        "data": "synthetic",
        "config": {"workload": workload, "dw_dtype": "bf16" if a.dw_bf16 else "f32",
                   "h_table": bool(a.h_table and p["kind"] != "linear"),
                   "pairs": r.N, "kept_pairs": M, "active_experts": int(np.count_nonzero(Me))},
        "roofline": roof,
        "gemm_kernels": ({k: {"ms": round(v["ms"], 4), "bytes": v["bytes"], "flops": v["flops"],
                              "gbs": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1),
                              "tflops": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2),
                              "pct_attainable": round(
                                  100 * v["flops"] / (v["ms"] * 1e-3) / 1e12
                                  / attainable_tflops(v["flops"] / v["bytes"], peak_tf), 2)}
                          for k, v in kernels.items()} if kernels else None),
        "grouped_gemm": {"ms": round(t_g * 1e3, 4), "tflops": round(tflops, 2),
                         "pct_mfma_peak": round(100 * tflops / peak_tf, 2),
                         "pct_attainable": round(100 * tflops / attainable_tflops(ai, peak_tf), 2),
                         "gbs": round(gbs, 1), "flops": flops, "bytes": gbytes,
                         "arith_intensity": round(ai, 1)},
        "stages_ms": {s: round(v, 4) for s, v in per.items()},
        "stages_gbs": {s: round(work[s]["bytes"] / (per[s] * 1e-3) / 1e9, 1) for s in mem_stages},
        "copy_gbs": round(cgbs, 1),
        "stages_frac_of_copy": {s: round(work[s]["bytes"] / (per[s] * 1e-3) / 1e9 / cgbs, 3)
                                for s in mem_stages},
        "score_compact_gbs": round(sum(work[s]["bytes"] for s in sc)
                                   / (sum(per[s] for s in sc) * 1e-3) / 1e9, 1),
        "unpruned_ms_per_step": round(ms_full, 4) if ms_full else None,
        "kept_fraction": round(M / r.N, 4),
        "pruned_over_unpruned_time": round(wall * 1e3 / ms_full, 4) if ms_full else None,
    }
    if not a.no_cpu:
        log("bench: timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(p, M, Me)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
