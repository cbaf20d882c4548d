"""Benchmark of the LRM-pruned MoE expert backward on one MI355X.

One step = one pass of the whole hot path over one layer call of synthetic
input already resident in HBM, through the fused C-ABI call: LRM score ->
per-expert top-quota select -> compaction -> grouped GEMM (dW, dX rows) ->
unpermute to token layout; SwiGLU workloads chain down -> gate/up stages.

The default workload is the largest single-GPU one, the heavy-skew SwiGLU
expert layer (T=65536, H=4096, I=1408, E=128, top-8, Zipf 1.6, bf16, fp32
weight gradients, per-expert caps keeping 0.1-1.0 of each expert's pairs).

Prints ONE JSON line.  `value` is kept pairs per second of the fused call
(for SwiGLU, pairs kept by the down stage), over K plain fused calls.  Stage
times come from a second pass of K calls in which the library records HIP
events on its launch stream at stage boundaries, one boundary after every
grouped-GEMM launch, so each launch has its own average duration.  The
`roofline` block covers the dominant kernel, the longest grouped-GEMM launch
of the call: its algorithmic flops (or bytes, below the ridge) over its
average duration from those events; `traffic` and `mfma_util` come from the
committed counter runs (profiles/gemm_counters.json) when they were taken on
this workload and this GEMM source.  The unpruned call (LRM_KEEP_ALL: every
pair kept, no score or select) is timed beside it, and the `cpu_baseline`
block times the fp64 CPU oracle on a stated sample.

    python bench.py [--steps K] [--warmup W] [--config 5] [--no-cpu] [--no-full]

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

The counter record the `roofline` fields read is written on any host, without
a GPU, from profiler passes over `--copy-probe --no-full` runs:

    python bench.py --record-counters FETCH_DIR WRITE_DIR [MFMA_DIR] [--config 5]
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
DEFAULT_CONFIG = 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG)
    ap.add_argument("--variant", default=None, help="3b: a real gate/up second selection")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-full", action="store_true",
                    help="skip the unpruned (keep-all) call, e.g. in profiler runs whose "
                         "kernel statistics should be those of the pruned call alone")
    ap.add_argument("--full", action="store_true", help=argparse.SUPPRESS)  # the default now
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain 512 MiB device copy (a known-size kernel that "
                         "calibrates the HBM byte counters of a profiler pass)")
    ap.add_argument("--h-table", action="store_true",
                    help="SwiGLU: pass the per-pair |silu(a) b|^2 a forward pass would save "
                         "(computed before timing), so the down score reads no A/B rows")
    ap.add_argument("--dw-bf16", action="store_true",
                    help="weight gradients stored as bf16 (LRM_DW_BF16) instead of fp32")
    ap.add_argument("--gather", action="store_true",
                    help="LRM_GATHER_LOADS: the w*x operand of the weight-gradient GEMMs is "
                         "gathered by their loaders instead of packed by compaction")
    ap.add_argument("--controller", action="store_true",
                    help="compare the workload's quotas with water-filling quotas of equal budget")
    ap.add_argument("--redistribute", action="store_true",
                    help="time the redistribution onto replicas instead of the bench line")
    ap.add_argument("--sweep", action="store_true",
                    help="keep-ratio sweep (quota = floor(r n_e)) instead of the bench line")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 --kernel-trace --stats run of "
                         "this bench (same --config/--steps/--warmup): every grouped-GEMM "
                         "launch of the pruned calls on its own, and the kernel statistics "
                         "(no GPU needed)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print a markdown table of rocprofv3 --pmc passes (GEMM_COUNTER_PASSES, "
                         "one folder each) over `bench.py --no-cpu --no-full` with the same "
                         "--config: stall, LDS, L1/L2 latency and TLB ratios per grouped-GEMM "
                         "launch (no GPU needed)")
    ap.add_argument("--record-counters", nargs="+", metavar="DIR",
                    help="write profiles/gemm_counters.json from the output folders of a "
                         "rocprofv3 --pmc FETCH_SIZE pass, a --pmc WRITE_SIZE pass and "
                         "optionally a --pmc MfmaUtil pass over `bench.py --no-cpu --no-full "
                         "--copy-probe` (no GPU needed)")
    return ap.parse_args()


COPY_KIB = 512 * 1024  # bytes moved each way by one copy of copy_probe, in KiB
COUNTERS_PATH = os.path.join(ROOT, "profiles", "gemm_counters.json")
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


def gemm_roles(kind, pass_through, fused=False):
    """The grouped-GEMM launches of one fused call, in launch order."""
    if kind == "linear":
        return ["gemm_dW", "gemm_dX"]
    if fused:
        return ["gemm_down_dW", "gemm_down_dX", "gemm_gateup_dW", "gemm_gateup_dX"]
    if pass_through:
        return ["gemm_down_dW", "gemm_down_dX", "gemm_gate_dW", "gemm_gate_dX", "gemm_up_dW"]
    return ["gemm_down_dW", "gemm_down_dX", "gemm_gate_dW", "gemm_gate_dX", "gemm_up_dW",
            "gemm_up_dX"]


def glu_pass_through(p):
    """The gate/up selections keep every down-kept row (one shared dX launch)."""
    return bool(np.all(np.asarray(p["quota_gate"]) >= np.asarray(p["quota_down"]))
                and np.all(np.asarray(p["quota_up"]) >= np.asarray(p["quota_down"])))


def glu_gate_up_fused(dtype, I, pass_through, gather=False):
    """One launch computes both gate/up weight gradients: pass-through, bf16
    inputs, I a multiple of 64, packed w x (no gathering loaders), unless
    LRM_FUSE_GATE_UP=0."""
    return (pass_through and dtype == "bf16" and I % 64 == 0 and not gather
            and not os.environ.get("LRM_FUSE_GATE_UP", "1").startswith("0"))


def workload_of(cfg, variant=None):
    """Workload name and the per-launch algorithmic work of one pruned call,
    from the routing and the quotas alone (no GPU)."""
    from pruned_expert_backward_lrm_amd import synth
    spec = synth.CONFIGS[cfg]
    r = synth.make_routing(spec["T"], spec["E"], spec["k"], spec["zipf"], "cfg", cfg,
                           local=spec.get("local"))
    q = synth._quotas(cfg, r, variant)
    b = 2 if spec["dtype"] == "bf16" else 4
    if spec["kind"] == "linear":
        shape = f"T={r.T} d_in={spec['d_in']} d_out={spec['d_out']}"
        Me = np.minimum(q["quota"], r.counts).astype(np.int64)
        work = gemm_launch_work("linear", r.E, b, 4, Me, d_in=spec["d_in"], d_out=spec["d_out"])
        return workload_name(spec, r.T, r.E, r.k, shape, variant), work, gemm_roles("linear", True)
    shape = f"T={r.T} H={spec['H']} I={spec['I']}"
    Md = np.minimum(q["quota_down"], r.counts).astype(np.int64)
    Mg = np.minimum(q["quota_gate"], Md)
    Mu = np.minimum(q["quota_up"], Md)
    pt = glu_pass_through(q)
    fused = glu_gate_up_fused(spec["dtype"], spec["I"], pt)
    work = gemm_launch_work("swiglu", r.E, b, 4, Md, Mg, Mu, H=spec["H"], I=spec["I"],
                            pass_through=pt, fused=fused)
    return (workload_name(spec, r.T, r.E, r.k, shape, variant), work,
            gemm_roles("swiglu", pt, fused))


def gemm_launch_work(kind, E, b, wb, Md, Mg=None, Mu=None, d_in=0, d_out=0, H=0, I=0,
                     pass_through=True, fused=False):
    """Algorithmic bytes and flops of each grouped-GEMM launch of one call.
    A dW launch writes every expert's dW (wb bytes an element) and reads its
    packed operands once; a dX launch reads W of the experts that kept rows
    and its packed gradient rows once, and writes the fp32 dX rows."""
    def dw(M, do, di):
        return dict(bytes=E * do * di * wb + int(M.sum()) * (di + do) * b,
                    flops=2.0 * int(M.sum()) * di * do)

    def dx(M, do, di, nseg=1):
        act = int(np.count_nonzero(M))
        return dict(bytes=nseg * (act * do * di * b + int(M.sum()) * do * b)
                    + int(M.sum()) * di * 4,
                    flops=2.0 * nseg * int(M.sum()) * di * do)

    if kind == "linear":
        return {"gemm_dW": dw(Md, d_out, d_in), "gemm_dX": dx(Md, d_out, d_in)}
    w = {"gemm_down_dW": dw(Md, H, I), "gemm_down_dX": dx(Md, H, I)}
    if fused:  # both weight gradients in one launch (2I rows), then both dX terms
        w["gemm_gateup_dW"] = dw(Md, 2 * I, H)
        w["gemm_gateup_dX"] = dx(Md, I, H, nseg=2)
        return w
    w.update({"gemm_gate_dW": dw(Mg, I, H), "gemm_up_dW": dw(Mu, I, H)})
    if pass_through:
        w["gemm_gate_dX"] = dx(Md, I, H, nseg=2)   # gate and up in one launch, K = 2I
    else:
        w["gemm_gate_dX"] = dx(Mg, I, H)
        w["gemm_up_dX"] = dx(Mu, I, H)
    return w


def is_gemm_kernel(name):
    """A grouped-GEMM kernel of the library (register path, LDS-DMA or fp32)."""
    return any(k in name for k in ("k_gemm_stream", "k_gemm_dma", "k_grouped_gemm"))


# Counter passes for --summarize-counters (each within one pass's limits)
GEMM_COUNTER_PASSES = [
    "SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT "
    "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_PENDING_STALL_CYCLES_sum "
    "TCP_UTCL1_STALL_INFLIGHT_MAX_sum TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
    "TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_TRANSLATION_HIT_sum TCC_EA0_RDREQ_LEVEL_sum "
    "TCC_EA0_RDREQ_sum GRBM_GUI_ACTIVE",
]


def summarize_counters(dirs, cfg, variant=None):
    """Markdown table of the GEMM_COUNTER_PASSES over `bench.py --no-cpu
    --no-full` (any order of folders): per grouped-GEMM launch of the pruned
    call (dispatches in launch order, as in record_counters), ratios of the
    per-dispatch means.  Per-CU fractions divide by the active cycles of one
    XCD (GRBM_GUI_ACTIVE, which the csv sums over the 8 XCDs when it reads
    more than 8 cycles per ns of dispatch) times the 256 CUs."""
    import csv
    import glob

    workload, work, roles = workload_of(cfg, variant)
    mean = {role: {} for role in roles}
    names = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        rows = [r for f in files for r in csv.DictReader(open(f))
                if is_gemm_kernel(r["Kernel_Name"])]
        by_counter = {}
        for r in rows:
            by_counter.setdefault(r["Counter_Name"], []).append(r)
        for counter, rs in by_counter.items():
            rs.sort(key=lambda r: int(r["Dispatch_Id"]))
            if len(rs) % len(roles):
                raise SystemExit(f"{d}: {len(rs)} dispatches of {counter}, not whole calls")
            for i, role in enumerate(roles):
                vals = [float(r["Counter_Value"]) for r in rs[i::len(roles)]]
                ns = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs[i::len(roles)]]
                key = counter if counter != "GRBM_GUI_ACTIVE" else f"GRBM_GUI_ACTIVE@{d}"
                mean[role][key] = float(np.mean(vals))
                mean[role].setdefault("ns", float(np.mean(ns)))
                names[role] = rs[i]["Kernel_Name"].split("(")[0].replace("lrm::", "").replace(
                    "void ", "")

    def cycles(m):
        g = [v for k, v in m.items() if k.startswith("GRBM_GUI_ACTIVE@")]
        if not g:
            return None
        c = float(np.mean(g))
        return c / 8 if c / m["ns"] > 8 else c

    def ratio(m, a, b, scale=100.0):
        return f"{scale * m[a] / m[b]:.1f}" if a in m and b in m and m[b] else "–"

    out = [f"Workload: {workload}.  Per grouped-GEMM launch of the pruned call, means "
           "over its dispatches:", "",
           "| launch | kernel | wait (any) % of wave cycles | LDS wait % | LDS issue % | "
           "LDS bank conflicts | MFMA busy % | L1 stalled on L2 % of CU cycles | "
           "L1 in-flight counter saturated % | L1→L2 reads | mean L1→L2 read latency "
           "(cycles) | L2 hit % | mean L2→memory read latency (cycles) | TLB misses / hits |",
           "|" + "---|" * 14]
    for role in roles:
        m = mean[role]
        cyc = cycles(m)
        cu = (lambda k: f"{100 * m[k] / (cyc * 256):.1f}" if k in m and cyc else "–")
        mfma = f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.1f}" \
            if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in m else "–"
        hit = (f"{100 * m['TCC_HIT_sum'] / (m['TCC_HIT_sum'] + m['TCC_MISS_sum']):.1f}"
               if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m else "–")
        tlb = (f"{m['TCP_UTCL1_TRANSLATION_MISS_sum']:.0f} / "
               f"{m['TCP_UTCL1_TRANSLATION_HIT_sum']:.3g}"
               if "TCP_UTCL1_TRANSLATION_MISS_sum" in m else "–")
        reqs = f"{m['TCP_TCC_READ_REQ_sum']:.3g}" if "TCP_TCC_READ_REQ_sum" in m else "–"
        out.append(
            f"| {role} | `{names.get(role, '?')}` | "
            f"{ratio(m, 'SQ_WAIT_INST_ANY', 'SQ_WAVE_CYCLES')} | "
            f"{ratio(m, 'SQ_WAIT_INST_LDS', 'SQ_WAVE_CYCLES')} | "
            f"{ratio(m, 'SQ_ACTIVE_INST_LDS', 'SQ_WAVE_CYCLES')} | "
            f"{m.get('SQ_LDS_BANK_CONFLICT', float('nan')):.0f} | {mfma} | "
            f"{cu('TCP_PENDING_STALL_CYCLES_sum')} | {cu('TCP_UTCL1_STALL_INFLIGHT_MAX_sum')} | "
            f"{reqs} | {ratio(m, 'TCP_TCC_READ_REQ_LATENCY_sum', 'TCP_TCC_READ_REQ_sum', 1.0)} | "
            f"{hit} | {ratio(m, 'TCC_EA0_RDREQ_LEVEL_sum', 'TCC_EA0_RDREQ_sum', 1.0)} | {tlb} |")
    print("\n".join(out))


def record_counters(dirs, cfg, variant=None):
    """profiles/gemm_counters.json from counter passes: per grouped-GEMM launch
    of the call, the average FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    scaled by what the same counter reads for the three 512 MiB copies of
    --copy-probe, and (third pass, optional) the average MfmaUtil.  The
    dispatches of each fused call come in launch order (gemm_roles)."""
    import csv
    import glob

    workload, work, roles = workload_of(cfg, variant)
    counters = ["FETCH_SIZE", "WRITE_SIZE", "MfmaUtil"][:len(dirs)]
    per = {role: {} for role in roles}
    names, scale = {}, {}
    for counter, d in zip(counters, dirs):
        rows = [row for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                                       recursive=True)
                for row in csv.DictReader(open(f)) if row["Counter_Name"] == counter]
        rows.sort(key=lambda row: int(row["Dispatch_Id"]))
        if counter != "MfmaUtil":
            copies = [float(row["Counter_Value"]) for row in rows
                      if row["Kernel_Name"] == "__amd_rocclr_copyBuffer"][:3]
            if len(copies) != 3:
                raise SystemExit(f"{d}: no --copy-probe copies found for {counter}")
            scale[counter] = float(np.mean(copies)) / COPY_KIB
        gemm = [row for row in rows if is_gemm_kernel(row["Kernel_Name"])]
        if not gemm or len(gemm) % len(roles):
            raise SystemExit(f"{d}: {len(gemm)} grouped-GEMM dispatches, not a whole number "
                             f"of calls of {len(roles)} launches")
        for i, role in enumerate(roles):
            vals = [float(row["Counter_Value"]) for row in gemm[i::len(roles)]]
            names[role] = gemm[i]["Kernel_Name"]
            per[role][counter] = (float(np.mean(vals)), len(vals))
    sha = gemm_source_sha()
    launches = []
    for role in roles:
        fk, n = per[role]["FETCH_SIZE"]
        wk, _ = per[role]["WRITE_SIZE"]
        fb = fk / scale["FETCH_SIZE"] * 1024
        wbytes = wk / scale["WRITE_SIZE"] * 1024
        alg = work[role]["bytes"]
        e = {"launch": role, "profiler_name": names[role], "workload": workload,
             "source_sha256": sha, "dispatches": n,
             "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
             "fetch_bytes": int(round(fb)), "write_bytes": int(round(wbytes)),
             "hbm_bytes": int(round(fb + wbytes)), "algorithmic_bytes": int(alg),
             "traffic_over_algorithmic": round((fb + wbytes) / alg, 3),
             "algorithmic_flops": work[role]["flops"]}
        if "MfmaUtil" in per[role]:
            e["mfma_util_pct"] = round(per[role]["MfmaUtil"][0], 2)
        launches.append(e)
    try:
        with open(COUNTERS_PATH) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    keep = [e for e in rec.get("launches", []) if e.get("workload") != workload]
    cmd_tail = f"--config {cfg}{' --variant ' + variant if variant else ''}"
    rec = {
        "note": ("Per grouped-GEMM launch of the fused call: HBM bytes from rocprofv3 --pmc "
                 "passes (FETCH_SIZE, WRITE_SIZE, KiB per dispatch) scaled by what the same "
                 "counter reads for a 512 MiB device copy in the same run, and the average "
                 "MfmaUtil (MFMA busy cycles over GPU active cycles and SIMDs, %).  "
                 "source_sha256 is the SHA-256 of csrc/k_gemm.hip, comments and whitespace "
                 "removed, that the counters were taken on."),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d FETCH_DIR -o run -- python "
            f"bench.py {cmd_tail} --no-cpu --no-full --copy-probe --steps 3 --warmup 1",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d WRITE_DIR -o run -- python "
            f"bench.py {cmd_tail} --no-cpu --no-full --copy-probe --steps 3 --warmup 1",
            "rocprofv3 --pmc MfmaUtil --output-format csv -d MFMA_DIR -o run -- python "
            f"bench.py {cmd_tail} --no-cpu --no-full --copy-probe --steps 3 --warmup 1",
            f"python bench.py {cmd_tail} --record-counters FETCH_DIR WRITE_DIR MFMA_DIR",
        ],
        "launches": keep + launches,
    }
    with open(COUNTERS_PATH, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps({"workload": workload, "launches": launches}, indent=1))


def summarize_trace(d, cfg, steps, warmup, variant=None):
    """Markdown summary of a kernel-trace run of this bench: the dispatches of
    the grouped-GEMM kernels come in calls of len(gemm_roles) launches; the
    first warmup + 2 * steps calls are the pruned ones (plain, then with
    stage events), so each launch of the pruned call gets its own average
    duration, comparable with the events of the bench line."""
    import csv
    import glob

    workload, work, roles = workload_of(cfg, variant)
    trace = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    stats = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if not trace:
        raise SystemExit(f"{d}: no kernel trace")
    rows = [r for f in trace for r in csv.DictReader(open(f))]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    gemm = [r for r in rows if is_gemm_kernel(r["Kernel_Name"])]
    ncalls = warmup + 2 * steps
    pruned = gemm[:ncalls * len(roles)]
    if len(pruned) != ncalls * len(roles):
        raise SystemExit(f"{d}: {len(gemm)} grouped-GEMM dispatches, fewer than {ncalls} calls")
    out = [f"Workload: {workload}.", "",
           f"Each pruned call makes {len(roles)} grouped-GEMM launches; the first {ncalls} "
           f"calls of the run ({warmup} warm-up, {steps} plain, {steps} with stage events) "
           "are pruned calls.  Per launch (kernel trace, end minus start of each dispatch):", "",
           "| launch | kernel | dispatches | avg µs | min µs | max µs | algorithmic TFLOP/s "
           "at avg | % of 2.5 PF |", "|---|---|---|---|---|---|---|---|"]
    for i, role in enumerate(roles):
        ds = pruned[i::len(roles)]
        us = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in ds])
        name = ds[0]["Kernel_Name"].replace("lrm::", "").replace("void ", "")
        tf = work[role]["flops"] / (us.mean() * 1e-6) / 1e12
        out.append(f"| {role} | `{name}` | {us.size} | {us.mean():.1f} | {us.min():.1f} | "
                   f"{us.max():.1f} | {tf:.1f} | {100 * tf / PEAK_TFLOPS['bf16']:.1f} |")
    if stats:
        out += ["", "Kernel statistics of the whole run (`*_kernel_stats.csv`, library "
                "kernels, every call of the run including the unpruned ones):", "",
                "| kernel | calls | avg µs | min µs | max µs | % of GPU time |",
                "|---|---|---|---|---|---|"]
        srows = [r for r in csv.DictReader(open(stats[0])) if "lrm::" in r["Name"]]
        for r in srows[:16]:
            name = r["Name"].replace("lrm::", "").replace("void ", "")
            out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                       f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                       f"{float(r['Percentage']):.2f} |")
    print("\n".join(out))


def counters_of(role, workload):
    """The committed counter record of one launch, or None when it was taken on
    another workload or another version of the GEMM source."""
    try:
        with open(COUNTERS_PATH) as f:
            rec = json.load(f)
        sha = gemm_source_sha()
    except (OSError, ValueError):
        return None
    for e in rec.get("launches", []):
        if e.get("launch") == role and e.get("workload") == workload \
                and e.get("source_sha256") == sha:
            return e
    return None


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

    def __init__(self, L, p, dev, dw_bf16=False, h_table=False, gather=False):
        self.L, self.p, self.r = L, p, p["routing"]
        self.dwb = dw_bf16
        self.gather = gather
        self.htab = None
        if h_table and p["kind"] != "linear":
            # what a forward pass would save: |silu(a) b|^2 per pair, fp64
            A, B = p["A"], p["B"]
            self.htab = torch.empty(A.shape[0], dtype=torch.float64, device=dev)
            for i in range(0, A.shape[0], 1 << 16):
                a, b = A[i:i + (1 << 16)].float(), B[i:i + (1 << 16)].float()
                h = a * torch.sigmoid(a) * b
                self.htab[i:i + (1 << 16)] = (h * h).sum(dim=1, dtype=torch.float64)
        fl = (L.LRM_DW_BF16 if dw_bf16 else 0) | (L.LRM_GATHER_LOADS if gather else 0)
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
            self.pass_through = True
            # the spans between the library's stage boundaries (lrm.h)
            self.stages = ["score", "select", "compact", "gemm_dW", "gemm_dX", "unpermute"]
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
                            dW_down=torch.empty(r.E, H, I, **wd), dX=torch.empty(r.T, H, **f32),
                            offsets_gate=torch.empty(r.E + 1, **i32),
                            offsets_up=torch.empty(r.E + 1, **i32))
            self.pass_through = glu_pass_through(p)
            self.fused = glu_gate_up_fused(p["dtype"], I, self.pass_through, gather)
            # one span per pair of consecutive boundaries; None: boundaries that
            # coincide (the fused gate/up launches leave two such spans)
            gu = (["gemm_gateup_dW", "gemm_gateup_dX", None, None] if self.fused else
                  ["gemm_gate_dW", "gemm_gate_dX", "gemm_up_dW", "gemm_up_dX"])
            self.stages = ["score_down", "select_down", "compact_down", "gemm_down_dW",
                           "gemm_down_dX", "glu_bwd", "select_gate_up", "compact_gate_up",
                           *gu, "unpermute"]
        if self.kind == "linear":
            self.fused = False
        self.gemm_roles = gemm_roles(self.kind, self.pass_through, self.fused)
        self.out["offsets"] = torch.empty(r.E + 1, **i32)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.ws = torch.empty(L.lrm_workspace_size(self.pb), **u8)
        self.ws_full = None
        self.out_full = dict(self.out)
        self.out_full["offsets"] = torch.empty(r.E + 1, **i32)

    def step(self, events=None):
        if events is None:
            self.L.lrm_expert_backward(self.pb, self.out, ws=self.ws)
        else:
            self.L.lrm_expert_backward_events(self.pb, self.out, events, ws=self.ws)

    def step_full(self):
        if self.ws_full is None:
            self.ws_full = torch.empty(self.L.lrm_workspace_size(self.pb_full), dtype=torch.uint8,
                                       device=self.ws.device)
        self.L.lrm_expert_backward(self.pb_full, self.out_full, ws=self.ws_full)

    def kept(self):
        """Kept rows per expert of the last pruned call: down (or the single
        projection), gate, up."""
        torch.cuda.synchronize()
        d = lambda k: np.diff(self.out[k].cpu().numpy().astype(np.int64))  # noqa: E731
        Me = d("offsets")
        if self.kind == "linear":
            return Me, Me, Me
        return Me, d("offsets_gate"), d("offsets_up")

    def work(self, Md, Mg, Mu):
        """Algorithmic bytes (and flops) of each stage: what the method must
        move, with the packed rows counted once and fp32 outputs."""
        p, r = self.p, self.r
        b = self.p["X"].element_size()
        wb = 2 if self.dwb else 4  # bytes of a stored weight-gradient element
        E, N, T = r.E, r.N, r.T
        M = int(Md.sum())
        if self.kind == "linear":
            di, do = p["d_in"], p["d_out"]
            xr = T if p["X_rows"] == "token" else N
            gr = T if p["G_rows"] == "token" else N
            w = {
                "score": dict(bytes=(xr * di + gr * do) * b + N * 12),
                "select": dict(bytes=N * 8 + M * 4),
                "compact": dict(bytes=2 * M * do * b + M * 8 if self.gather
                                else 2 * M * (di + do) * b),
                "unpermute": dict(bytes=M * di * 4 + T * di * 4),
            }
            w.update(gemm_launch_work("linear", E, b, wb, Md, d_in=di, d_out=do))
            return w
        H, I = p["H"], p["I"]
        Mgs, Mus = int(Mg.sum()), int(Mu.sum())
        w = {
            "score_down": dict(bytes=T * H * b + (N * 8 if self.htab is not None else 2 * N * I * b)
                               + N * 12),
            "select_down": dict(bytes=N * 8 + M * 4),
            "compact_down": dict(bytes=2 * M * H * b + 3 * M * I * b),
            "glu_bwd": dict(bytes=T * H * b + M * I * 4 + 4 * M * I * b),
            "select_gate_up": dict(bytes=2 * (M * 8) + (Mgs + Mus) * 4),
            "compact_gate_up": dict(bytes=(M * 8 if self.gather else 2 * M * H * b)
                                    if self.pass_through
                                    else 2 * (Mgs + Mus) * ((0 if self.gather else H) + I) * b
                                    + ((Mgs + Mus) * 8 if self.gather else 0)),
            "unpermute": dict(bytes=M * H * 4 * (1 if self.pass_through else 2) + T * H * 4),
        }
        w.update(gemm_launch_work("swiglu", E, b, wb, Md, Mg, Mu, H=H, I=I,
                                  pass_through=self.pass_through, fused=self.fused))
        return w


def time_fused(W, steps, warmup):
    """Wall time per step of the plain fused call (the timed region holds the
    steps only), then the per-stage split from a second pass of the same
    steps with HIP events recorded by the library at its stage boundaries,
    one after every grouped-GEMM launch (the events cost a little GPU time of
    their own, so they stay out of the first pass)."""
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
           for i, name in enumerate(W.stages) if name is not None}
    return wall, per, wall_ev


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
    # sample of experts (every third by kept rows, largest first) holding
    # about a third of the kept rows
    host = dict(p, **{k: p[k].cpu() for k in ("X", "G", "A", "B", "W_gate", "W_up", "W_down")})
    order = np.argsort(Me, kind="stable")
    ex, tot = [], 0
    for e in order[::-1][::3]:
        if tot >= M / 3:
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
    if a.summarize_trace:
        summarize_trace(a.summarize_trace, a.config, a.steps, a.warmup, a.variant)
        return
    if a.summarize_counters:
        summarize_counters(a.summarize_counters, a.config, a.variant)
        return
    if a.record_counters:
        if not 2 <= len(a.record_counters) <= 3:
            raise SystemExit("--record-counters FETCH_DIR WRITE_DIR [MFMA_DIR]")
        record_counters(a.record_counters, a.config, a.variant)
        return
    if a.gpus != 1:
        log("bench.py: the library runs one GPU's share of the experts on one GPU "
            "(the collectives across GPUs are not part of it); --gpus must be 1")
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
    W = Workload(L, p, dev, a.dw_bf16, a.h_table, a.gather)
    r = p["routing"]
    log("bench: timing the pruned backward")
    wall, per, wall_ev = time_fused(W, a.steps, a.warmup)
    Md, Mg, Mu = W.kept()
    M = int(Md.sum())
    ms_full = None
    if not a.no_full:
        log("bench: timing the unpruned backward (every pair kept)")
        ms_full = time_loop(W.step_full, a.steps, a.warmup) * 1e3
        W.ws_full = None
        torch.cuda.empty_cache()
    work = W.work(Md, Mg, Mu)
    roles = W.gemm_roles
    flops = sum(work[s]["flops"] for s in roles)
    gbytes = sum(work[s]["bytes"] for s in roles)
    gemm_stages = [s for s in per if s.startswith("gemm_")]
    t_g = sum(per[s] for s in gemm_stages) * 1e-3
    ai = flops / gbytes
    peak_tf = PEAK_TFLOPS[p["dtype"]]
    ridge = peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
    tflops = flops / t_g / 1e12
    spec = synth.CONFIGS[a.config]
    if p["kind"] == "linear":
        shape = f"T={r.T} d_in={p['d_in']} d_out={p['d_out']}"
    else:
        shape = f"T={r.T} H={p['H']} I={p['I']}"
    workload = workload_name(spec, r.T, r.E, r.k, shape, a.variant)
    launches = {}
    for role in roles:
        t = per[role] * 1e-3
        w = work[role]
        launches[role] = {"ms": round(per[role], 4), "flops": w["flops"], "bytes": w["bytes"],
                          "tflops": round(w["flops"] / t / 1e12, 2),
                          "pct_mfma_peak": round(100 * w["flops"] / t / 1e12 / peak_tf, 2),
                          "gbs": round(w["bytes"] / t / 1e9, 1),
                          "pct_attainable": round(100 * w["flops"] / t / 1e12 / attainable_tflops(
                              w["flops"] / w["bytes"], peak_tf), 2)}
    # the dominant kernel: the longest grouped-GEMM launch of the call
    dom = max(roles, key=lambda k: per[k])
    kd, k_t = work[dom], per[dom] * 1e-3
    rec = counters_of(dom, workload) if not (a.dw_bf16 or a.h_table or a.gather) else None
    if kd["flops"] / kd["bytes"] < ridge:
        k_gbs = kd["bytes"] / k_t / 1e9
        roof = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(k_gbs / PEAK_HBM_GBS, 4)}
    else:
        k_tf = kd["flops"] / k_t / 1e12
        roof = {"bound": "mfma", "achieved": round(k_tf, 2), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(k_tf / peak_tf, 4)}
    roof["traffic"] = rec["hbm_bytes"] if rec else None
    roof["kernel"] = dom
    roof["profiler_name"] = rec["profiler_name"] if rec else None
    roof["mfma_util_pct"] = rec.get("mfma_util_pct") if rec else None
    roof["algorithmic_flops"] = kd["flops"]
    roof["algorithmic_bytes"] = kd["bytes"]
    roof["launch_ms"] = round(per[dom], 4)
    mem_stages = [s for s in per if not s.startswith("gemm_") and s in work]
    log("bench: measuring device-copy bandwidth")
    cgbs = copy_gbs(dev)
    sc = [s for s in per if s.startswith("score") or s.startswith("compact")]
    gbs_of = lambda s: work[s]["bytes"] / (per[s] * 1e-3) / 1e9  # noqa: E731
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
                   "gather_loads": bool(a.gather),
                   "h_table": bool(a.h_table and p["kind"] != "linear"),
                   "pairs": r.N, "kept_pairs": M, "active_experts": int(np.count_nonzero(Md)),
                   **({} if p["kind"] == "linear" else
                      {"kept_gate": int(Mg.sum()), "kept_up": int(Mu.sum())})},
        "roofline": roof,
        "gemm_launches": launches,
        "grouped_gemm": {"ms": round(t_g * 1e3, 4), "tflops": round(tflops, 2),
                         "pct_mfma_peak": round(100 * tflops / peak_tf, 2),
                         "pct_attainable": round(100 * tflops / attainable_tflops(ai, peak_tf), 2),
                         "gbs": round(gbytes / t_g / 1e9, 1), "flops": flops, "bytes": gbytes,
                         "arith_intensity": round(ai, 1)},
        "stages_ms": {s: round(v, 4) for s, v in per.items()},
        "stages_gbs": {s: round(gbs_of(s), 1) for s in mem_stages},
        "stages_frac_of_hbm_peak": {s: round(gbs_of(s) / PEAK_HBM_GBS, 3) for s in mem_stages},
        "memory_stages_gbs": round(sum(work[s]["bytes"] for s in mem_stages)
                                   / (sum(per[s] for s in mem_stages) * 1e-3) / 1e9, 1),
        "score_compact_gbs": round(sum(work[s]["bytes"] for s in sc)
                                   / (sum(per[s] for s in sc) * 1e-3) / 1e9, 1),
        "copy_gbs": round(cgbs, 1),
        "unpruned_ms_per_step": round(ms_full, 4) if ms_full else None,
        "kept_fraction": round(M / r.N, 4),
        "pruned_over_unpruned_time": round(wall * 1e3 / ms_full, 4) if ms_full else None,
    }
    if not a.no_cpu:
        log("bench: timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(p, M, Md)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
