"""The unchanged library sources on the CPU: every kernel compiled as host C++
against tests/cpu_emu/cpu_emu.h (lanes as threads, wave collectives, buffer
range checks, an MFMA model) with AddressSanitizer, driven through the fused
C-ABI call by tests/cpu_emu/emu_driver.cpp.  Any out-of-bounds global-memory
access of a kernel or of the host code aborts the run; the outputs must pass
the same oracle checks as the GPU parity tests.  Runs without a GPU.

Every lane is an OS thread and every wave collective two 64-thread barriers,
so a case takes 30-150 s.  The default run keeps the tiny fp32 workload
(every step, the fp32 GEMM), the bf16 grouped GEMM in its 256x256 tiles,
the dW schedule with its tiles striped over the XCDs, the SwiGLU gate/up
weight gradients in one launch over two outputs, and the selection's error
and capacity cases; LRM_EMU_FULL=1 runs all of them, the opt-in LDS-DMA and
gathering kernels included (about 30 minutes on 8 cores, or 10 with
pytest -n 3).
"""

from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess

import numpy as np
import pytest
import torch

from pruned_expert_backward_lrm_amd import synth
from parity import judge_linear, judge_swiglu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "pruned_expert_backward_lrm_amd", "csrc")
EMU = os.path.join(ROOT, "tests", "cpu_emu")
CLANG = "/opt/rocm/llvm/bin/clang++"
# host quotas of more than QUOTA_PACK_MAX experts take the library's stream-copy
# path (512 in the product build; lowered here so that path runs on small E)
QUOTA_PACK_MAX = 8
# the bucketing's many-workgroup row scan runs from this many histogram
# counts (32768 in the product build; 1 here so every emulated call takes it)
BUCKET_ROWS_MIN = 1
FLAGS = ["-std=c++20", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
         f"-DLRM_QUOTA_PACK_MAX={QUOTA_PACK_MAX}", f"-DLRM_BUCKET_ROWS_MIN={BUCKET_ROWS_MIN}"]

LINEAR, SWIGLU = 0, 1
F32, BF16 = 0, 1
KEEP_ALL = 1
ROWS = {"token": 0, "pair": 1}

extended = pytest.mark.skipif(not os.environ.get("LRM_EMU_FULL"),
                              reason="extended emulation case (set LRM_EMU_FULL=1)")


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("clang++ of the ROCm toolchain not found")
    srcs = _sources() + [os.path.join(EMU, "emu_driver.cpp")]
    h = hashlib.sha256()
    for s in srcs + [os.path.join(EMU, "cpu_emu.h")] + \
            [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]:
        with open(s, "rb") as f:
            h.update(f.read())
    out = tmp_path_factory.mktemp("emu_" + h.hexdigest()[:12])

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        cmd = [CLANG, *FLAGS, "-DLRM_CPU_EMU", "-x", "c++", "-I", EMU, "-I",
               os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{src}:\n{r.stderr[-4000:]}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(out, "emu_driver")
    r = subprocess.run([CLANG, "-fsanitize=address", "-o", exe, *objs, "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def _raw(t: torch.Tensor) -> bytes:
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().tobytes()
    return t.numpy().tobytes()


def run_emu(exe, tmp_path, p: dict, flags: int = 0, env_extra=None, expect=(0, 0)) -> dict:
    """One fused call of the emulated library.  Returns the outputs as CPU
    tensors under the keys the GPU parity helpers use.  `expect`: the status
    of the call and of lrm_check_device_errors after it (-1: not run)."""
    r = p["routing"]
    N, E, T = r.N, r.E, r.T
    Nr = max(N, 1)
    dt = BF16 if p["dtype"] == "bf16" else F32
    kind = LINEAR if p["kind"] == "linear" else SWIGLU
    d_in = p.get("d_in", 0)
    d_out = p.get("d_out", 0)
    H, I = p.get("H", 0), p.get("I", 0)
    xr = ROWS[p.get("X_rows", "token")]
    gr = ROWS[p.get("G_rows", "token")]
    if kind == SWIGLU:
        Md = N if flags & KEEP_ALL else int(np.minimum(p["quota_down"], r.counts).sum())
        Md = max(Md, 1)
    else:
        Md = 0
    hdr = np.array([kind, dt, flags, T, N, E, d_in, d_out, H, I, xr, gr, Md, 0, 0, 0], np.int32)
    pad = lambda a, dtype: np.ascontiguousarray(  # noqa: E731
        np.concatenate([np.asarray(a, dtype), np.zeros(Nr - len(a), dtype)]))
    parts = [hdr.tobytes(), pad(r.token, np.int32).tobytes(), pad(r.expert, np.int32).tobytes(),
             pad(r.weight, np.float32).tobytes()]
    if kind == LINEAR:
        parts += [_raw(p["X"]), _raw(p["G"]), _raw(p["W"]),
                  np.asarray(p["quota"], np.int32).tobytes()]
    else:
        parts += [_raw(p[k]) for k in ("X", "G", "A", "B", "W_gate", "W_up", "W_down")]
        parts += [np.asarray(p[k], np.int32).tobytes()
                  for k in ("quota_down", "quota_gate", "quota_up")]
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(b"".join(parts))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    env.pop("LRM_GEMM_TILE", None)
    env.update(env_extra or {})
    res = subprocess.run([exe, str(fin), str(fout)], capture_output=True, text=True,
                         timeout=600, env=env)
    assert res.returncode == 0, f"emulated run failed ({res.returncode}):\n{res.stderr[-6000:]}"
    buf = fout.read_bytes()
    off = 0

    def take(n, dtype, shape=None):
        nonlocal off
        a = np.frombuffer(buf, dtype=dtype, count=n, offset=off).copy()
        off += n * np.dtype(dtype).itemsize
        return torch.from_numpy(a.reshape(shape) if shape else a)

    status, dev_status = (int(v) for v in take(2, np.int32))
    assert (status, dev_status) == tuple(expect), \
        f"lrm_expert_backward returned {status}, lrm_check_device_errors {dev_status}"
    out = {}
    if kind == LINEAR:
        out["dW"] = take(E * d_out * d_in, np.float32, (E, d_out, d_in))
        rows = T if xr == 0 else N
        out["dX"] = take(rows * d_in, np.float32, (rows, d_in))
    else:
        for k in ("dW_gate", "dW_up"):
            out[k] = take(E * I * H, np.float32, (E, I, H))
        out["dW_down"] = take(E * H * I, np.float32, (E, H, I))
        out["dX"] = take(T * H, np.float32, (T, H))
    out["score"] = take(Nr, np.float32)
    out["pos"] = take(Nr, np.int32)
    out["offsets"] = take(E + 1, np.int32)
    if kind == SWIGLU:
        out["score_gate"] = take(Md, np.float32)
        out["score_up"] = take(Md, np.float32)
        out["pos_gate"] = take(Md, np.int32)
        out["pos_up"] = take(Md, np.int32)
        out["offsets_gate"] = take(E + 1, np.int32)
        out["offsets_up"] = take(E + 1, np.int32)
        out["dH"] = take(Md * I, np.float32, (Md, I))
    assert off == len(buf)
    return out


def test_emu_linear_config1(driver, tmp_path):
    p = synth.make_config(1)
    judge_linear(p, run_emu(driver, tmp_path, p))


@extended
@pytest.mark.parametrize("x_rows,g_rows", [("token", "pair"), ("pair", "token")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_emu_linear_ragged(driver, tmp_path, dtype, x_rows, g_rows):
    # ragged feature sizes (not multiples of the tiles), skewed experts,
    # quotas that keep 0..all of an expert
    p = synth.make_linear(300, 10, 4, 136, 200, dtype=dtype, x_rows=x_rows, g_rows=g_rows,
                          seed=8, zipf=1.4, quota=lambda c: (c * 5) // 8 + (c % 3 == 0))
    judge_linear(p, run_emu(driver, tmp_path, p))


@pytest.mark.parametrize("tile", [pytest.param("S", marks=extended),
                                  pytest.param("M", marks=extended), "L",
                                  pytest.param("X", marks=extended)])
def test_emu_linear_tile_configs(driver, tmp_path, tile):
    # every bf16 tile configuration of the grouped GEMM, over an expert with
    # more rows than one 256-row tile and experts that keep nothing
    p = synth.make_linear(400, 4, 2, 72, 264, dtype="bf16", seed=3, zipf=1.6,
                          quota=lambda c: np.where(np.arange(c.size) == 3, 0, c))
    judge_linear(p, run_emu(driver, tmp_path, p, env_extra={"LRM_GEMM_TILE": tile}))


@pytest.mark.parametrize("dma", [pytest.param("2", marks=extended), pytest.param("4", marks=extended)])
def test_emu_gemm_lds_dma(driver, tmp_path, dma):
    """The 256x256 kernels whose operand tiles go straight into LDS and whose
    k-strided operands are read with transposing LDS reads (LRM_GEMM_DMA=2:
    k-tiles of 64 in two stages; 4: of 32 in four), dW and dX, on a ragged
    shape (a partial last column tile, an expert over several row tiles, one
    that keeps nothing): judged against the oracle and, with LRM_EMU_FULL=1,
    compared bit for bit with the register path (LRM_GEMM_DMA=0), which issues
    the same MFMAs in the same order on the same operands."""
    p = synth.make_linear(400, 4, 2, 200, 320, dtype="bf16", seed=3, zipf=1.6,
                          quota=lambda c: np.where(np.arange(c.size) == 3, 0, c))
    got = run_emu(driver, tmp_path, p, env_extra={"LRM_GEMM_TILE": "L", "LRM_GEMM_DMA": dma})
    judge_linear(p, got)
    if os.environ.get("LRM_EMU_FULL"):  # the bit-for-bit comparison costs a second run
        ref = run_emu(driver, tmp_path, p, env_extra={"LRM_GEMM_TILE": "L", "LRM_GEMM_DMA": "0"})
        for k in ("dW", "dX"):
            assert torch.equal(ref[k], got[k]), k


@pytest.mark.parametrize("tile", ["L", pytest.param("X", marks=extended)])
def test_emu_dw_heavy_stripes(driver, tmp_path, tile):
    """The dW schedule with heavy experts striped over the XCDs: 8 tiles per
    expert (512 x 1024 outputs of 256 x 256).  The total work is small, so
    every expert (an empty one included) counts as heavy and all tiles go
    out in stripes, past runs of the equal-cost cut that hold no tiles; one
    block per tile (L) and persistent blocks (X), under AddressSanitizer and
    judged against the oracle.  (A mix of heavy and light experts needs more
    work than the emulation affords; the GPU tests cover it.)"""
    p = synth.make_linear(240, 6, 1, 1024, 512, dtype="bf16", seed=12, zipf=1.8)
    judge_linear(p, run_emu(driver, tmp_path, p, env_extra={"LRM_GEMM_TILE": tile}))


@extended
def test_emu_linear_keep_all(driver, tmp_path):
    p = synth.make_linear(200, 6, 2, 64, 96, dtype="bf16", seed=4, zipf=0.8)
    judge_linear(p, run_emu(driver, tmp_path, p, flags=KEEP_ALL), keep_all=True)


@extended
@pytest.mark.parametrize("variant", ["same", "second"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_emu_swiglu(driver, tmp_path, dtype, variant):
    quotas = {
        "same": (lambda c: c // 2, lambda c: c // 2, lambda c: c // 2),
        "second": (lambda c: (3 * c) // 4, lambda c: (3 * c) // 8 + 1, lambda c: c // 3),
    }[variant]
    p = synth.make_swiglu(160, 6, 2, 136, 72, dtype=dtype, seed=5, zipf=1.2, quotas=quotas,
                          g_std=1e-2)
    judge_swiglu(p, run_emu(driver, tmp_path, p))


@pytest.mark.parametrize("tile", [pytest.param("S", marks=extended), "L",
                                  pytest.param("X", marks=extended)])
def test_emu_swiglu_fused_gate_up(driver, tmp_path, tile):
    """Gate and up keep the down stage's rows (same quotas), bf16, I = 192: one
    dW launch over [GA | GB] (2I = 384 rows per expert) writes rows below I to
    dW_gate and the rest to dW_up, a tile straddling the split (256-row tiles:
    rows 0..255 hold all of the gate rows and 64 up rows; 128-row tiles: the
    second one's waves write to either side), and the dX launch reads GA and
    GB as two K segments of the 2I-wide rows.  Under AddressSanitizer and
    judged against the oracle."""
    p = synth.make_swiglu(160, 6, 2, 72, 192, dtype="bf16", seed=5, zipf=1.2,
                          quotas=(lambda c: c // 2, lambda c: c // 2, lambda c: c // 2),
                          g_std=1e-2)
    judge_swiglu(p, run_emu(driver, tmp_path, p, env_extra={"LRM_GEMM_TILE": tile}))


def _no_pairs(kind, dtype, T=48, E=4):
    r = synth.Routing(T, E, 2, np.zeros(0, np.int32), np.zeros(0, np.int32),
                      np.zeros(0, np.float32), np.zeros(E, np.int64))
    dt = synth.torch_dtype(dtype)
    g = torch.Generator().manual_seed(13)
    q = np.full(E, 2, np.int32)
    if kind == "linear":
        return dict(kind="linear", dtype=dtype, routing=r, T=T, N=0, E=E, k=2, d_in=64,
                    d_out=32, X_rows="token", G_rows="token", quota=q,
                    X=torch.randn(T, 64, generator=g).to(dt),
                    G=torch.randn(T, 32, generator=g).to(dt),
                    W=torch.randn(E, 32, 64, generator=g).to(dt))
    H, I = 64, 32
    return dict(kind="swiglu", dtype=dtype, routing=r, T=T, N=0, E=E, k=2, H=H, I=I,
                quota_down=q, quota_gate=q.copy(), quota_up=q.copy(),
                X=torch.randn(T, H, generator=g).to(dt), G=torch.randn(T, H, generator=g).to(dt),
                A=torch.zeros(0, I).to(dt), B=torch.zeros(0, I).to(dt),
                W_gate=torch.randn(E, I, H, generator=g).to(dt),
                W_up=torch.randn(E, I, H, generator=g).to(dt),
                W_down=torch.randn(E, H, I, generator=g).to(dt))


@pytest.mark.parametrize("kind", ["linear", "swiglu"])
def test_emu_no_pairs(driver, tmp_path, kind):
    # no pair on this GPU: every output written, exactly zero
    p = _no_pairs(kind, "bf16")
    out = run_emu(driver, tmp_path, p)
    keys = ("dW", "dX") if kind == "linear" else ("dW_gate", "dW_up", "dW_down", "dX")
    for k in keys:
        assert not torch.any(out[k] != 0), f"{k} must be exactly zero"
    assert torch.equal(out["offsets"], torch.zeros(p["E"] + 1, dtype=torch.int32))


def test_emu_bad_expert_id(driver, tmp_path):
    # an expert id out of range: the pair is left out of every step, the call
    # returns LRM_OK and the device error word reports it (LRM_ERR_INDEX = 8);
    # with LRM_DEBUG_CHECKS (8) the call itself returns LRM_ERR_INDEX
    p = synth.make_linear(64, 4, 2, 32, 32, dtype="bf16", seed=9)
    r = p["routing"]
    r.expert = r.expert.copy()
    r.expert[5] = r.E + 3
    run_emu(driver, tmp_path, p, expect=(0, 8))
    run_emu(driver, tmp_path, p, flags=8, expect=(8, -1))


@pytest.mark.parametrize("kind", ["linear", "swiglu"])
def test_emu_selection_past_packed_capacity(driver, tmp_path, kind):
    """Host quotas of more than QUOTA_PACK_MAX experts are copied into the
    workspace on the stream.  The emulation adds 50 to every quota of that
    copy, as a captured call replayed after its host quota arrays grew would
    see: the selections then keep more rows than the host sized the packed
    buffers for.  Every access must stay in bounds (AddressSanitizer), the
    call must return LRM_OK and the device error word LRM_ERR_WORKSPACE (7);
    the kept counts are capped at the packed capacity."""
    E = 2 * QUOTA_PACK_MAX
    if kind == "linear":
        p = synth.make_linear(96, E, 2, 8, 8, dtype="f32", seed=21, zipf=2.0,
                              quota=lambda c: c // 4)
        cap = int(np.minimum(p["quota"], p["routing"].counts).sum())
    else:
        q = lambda c: c // 4  # noqa: E731
        p = synth.make_swiglu(96, E, 2, 8, 8, dtype="f32", seed=21, zipf=2.0,
                              quotas=(q, q, q), g_std=1e-2)
        cap = int(np.minimum(p["quota_down"], p["routing"].counts).sum())
    assert 0 < cap < p["routing"].N // 2
    out = run_emu(driver, tmp_path, p, env_extra={"LRM_EMU_H2D_INT_ADD": "50"}, expect=(0, 7))
    offs = out["offsets"].numpy().astype(np.int64)
    assert offs[-1] == cap and np.all(np.diff(offs) >= 0)
    if kind == "swiglu":
        for k in ("offsets_gate", "offsets_up"):
            assert out[k].numpy()[-1] <= cap


@extended
def test_emu_gather_loads(driver, tmp_path):
    """LRM_GATHER_LOADS (16) under AddressSanitizer: the dW loader that
    gathers and scales the x rows itself stays in bounds (a ragged k tail,
    experts that keep nothing) and gives the outputs of the packed path bit
    for bit."""
    p = synth.make_linear(400, 4, 2, 72, 264, dtype="bf16", x_rows="pair", g_rows="token",
                          seed=3, zipf=1.6, quota=lambda c: np.where(np.arange(c.size) == 3, 0, c))
    ref = run_emu(driver, tmp_path, p, env_extra={"LRM_GEMM_TILE": "L"})
    got = run_emu(driver, tmp_path, p, flags=16, env_extra={"LRM_GEMM_TILE": "L"})
    for k in ("dW", "dX", "score", "pos", "offsets"):
        assert torch.equal(got[k], ref[k]), k
