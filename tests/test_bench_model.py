"""The benchmark's accounting, on the CPU: the grouped-GEMM launches a call
makes and the algorithmic work each is credited with (the roofline of the
bench line divides by these), and the refusal of more than one GPU."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counts(seed=3, E=16):
    rng = np.random.default_rng(seed)
    Md = rng.integers(0, 700, E).astype(np.int64)
    Md[3] = 0  # an expert that keeps nothing
    return Md


def test_fused_gate_up_work_is_the_two_launches_minus_one_read():
    """One gate/up dW launch over 2I rows does the flops of the gate and up
    launches and reads the packed w x rows once instead of twice; its dX
    launch is the pass-through one (K = 2I in two segments)."""
    E, b, wb, H, I = 16, 2, 4, 512, 192
    Md = _counts(E=E)
    sep = bench.gemm_launch_work("swiglu", E, b, wb, Md, Md, Md, H=H, I=I, pass_through=True)
    fus = bench.gemm_launch_work("swiglu", E, b, wb, Md, Md, Md, H=H, I=I, pass_through=True,
                                 fused=True)
    M = int(Md.sum())
    assert fus["gemm_gateup_dW"]["flops"] == sep["gemm_gate_dW"]["flops"] + sep["gemm_up_dW"]["flops"]
    assert (fus["gemm_gateup_dW"]["bytes"]
            == sep["gemm_gate_dW"]["bytes"] + sep["gemm_up_dW"]["bytes"] - M * H * b)
    assert fus["gemm_gateup_dX"] == sep["gemm_gate_dX"]
    for k in ("gemm_down_dW", "gemm_down_dX"):
        assert fus[k] == sep[k]
    # dW: every expert's fp32 output plus the packed operands once; flops 2 M d_in d_out
    assert fus["gemm_gateup_dW"]["bytes"] == E * 2 * I * H * wb + M * (H + 2 * I) * b
    assert fus["gemm_gateup_dW"]["flops"] == 2.0 * M * H * 2 * I


def test_dx_reads_w_of_active_experts_only():
    E, b, wb = 16, 2, 4
    Md = _counts(E=E)
    w = bench.gemm_launch_work("linear", E, b, wb, Md, d_in=256, d_out=128)
    act = int(np.count_nonzero(Md))
    M = int(Md.sum())
    assert w["gemm_dX"]["bytes"] == act * 128 * 256 * b + M * 128 * b + M * 256 * 4
    assert w["gemm_dW"]["bytes"] == E * 128 * 256 * wb + M * (256 + 128) * b


@pytest.mark.parametrize("env,fused", [(None, True), ("0", False)])
def test_roles_follow_the_library_choice(monkeypatch, env, fused):
    """bf16 SwiGLU workloads with I a multiple of 64 and equal quotas run the
    gate/up weight gradients as one launch unless LRM_FUSE_GATE_UP=0, as the
    library does; the linear workload makes two launches."""
    if env is None:
        monkeypatch.delenv("LRM_FUSE_GATE_UP", raising=False)
    else:
        monkeypatch.setenv("LRM_FUSE_GATE_UP", env)
    _, work, roles = bench.workload_of(5)
    if fused:
        assert roles == ["gemm_down_dW", "gemm_down_dX", "gemm_gateup_dW", "gemm_gateup_dX"]
    else:
        assert roles == ["gemm_down_dW", "gemm_down_dX", "gemm_gate_dW", "gemm_gate_dX",
                         "gemm_up_dW"]
    assert set(roles) <= set(work)
    _, _, roles2 = bench.workload_of(2)
    assert roles2 == ["gemm_dW", "gemm_dX"]
    assert not bench.glu_gate_up_fused("f32", 1408, True)
    assert not bench.glu_gate_up_fused("bf16", 1400, True)
    assert not bench.glu_gate_up_fused("bf16", 1408, False)
    assert not bench.glu_gate_up_fused("bf16", 1408, True, gather=True)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr + r.stdout
