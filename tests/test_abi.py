"""The C-ABI library loads and exports what include/lrm.h declares; host-side
validation rejects bad arguments before any HIP call (no GPU needed)."""

import ctypes as C
import os
import re

import numpy as np
import pytest

from pruned_expert_backward_lrm_amd import lrm as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "lrm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lrm_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 16
    lib = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


def test_struct_layouts_match_header():
    # explicit padding in the header makes these sizes ABI-stable
    assert C.sizeof(L.lrm_pairs) == 40
    assert C.sizeof(L.lrm_mat) == 32
    assert C.sizeof(L.lrm_outputs) == 15 * 8
    assert L.lrm_problem.X.offset == 56 and L.lrm_problem.quota.offset == 144
    assert C.sizeof(L.lrm_problem) == 280 and L.lrm_problem.h_sumsq.offset == 272


def test_status_strings_and_version():
    for s in range(12):
        assert L._lib.lrm_status_string(s)
        assert L._lib.lrm_status_string(s) != b"unknown status"
    assert L._lib.lrm_status_string(999) == b"unknown status"
    assert L._lib.lrm_version() >= 100


def test_max_kept():
    q = np.array([3, 0, 5], np.int32)
    assert L.lrm_max_kept(100, q) == 8
    assert L.lrm_max_kept(6, q) == 6
    assert L.lrm_max_kept(6, np.array([1, -1], np.int32)) == -1


def _pairs(T=4, N=4, E=2, ptr=0x1000):
    return L.lrm_pairs(T, N, E, 0, ptr, ptr, ptr)


def _m(ptr=0x1000, dtype=L.LRM_BF16, rows=L.LRM_ROWS_TOKEN, cols=64, ld=64):
    return L.lrm_mat(ptr, dtype, rows, cols, 0, ld)


def test_score_validation_returns_before_launch():
    lib = L._lib
    ws, score = C.c_void_p(0x2000), C.c_void_p(0x3000)
    p = _pairs()
    X, G = _m(), _m(cols=32, ld=32)
    assert lib.lrm_score(None, C.byref(X), C.byref(G), score, ws, 1 << 20, None) == 1
    bad = _pairs(E=0)
    assert lib.lrm_score(C.byref(bad), C.byref(X), C.byref(G), score, ws, 1 << 20, None) == 2
    Xd = _m(dtype=L.LRM_F32)
    assert lib.lrm_score(C.byref(p), C.byref(Xd), C.byref(G), score, ws, 1 << 20, None) == 3
    Xl = _m(rows=7)
    assert lib.lrm_score(C.byref(p), C.byref(Xl), C.byref(G), score, ws, 1 << 20, None) == 4
    Xa = _m(ptr=0x1008)
    assert lib.lrm_score(C.byref(p), C.byref(Xa), C.byref(G), score, ws, 1 << 20, None) == 5
    Xc = _m(cols=60, ld=64)
    assert lib.lrm_score(C.byref(p), C.byref(Xc), C.byref(G), score, ws, 1 << 20, None) == 10
    Xs = _m(cols=64, ld=32)
    assert lib.lrm_score(C.byref(p), C.byref(Xs), C.byref(G), score, ws, 1 << 20, None) == 2
    assert lib.lrm_score(C.byref(p), C.byref(X), C.byref(G), score, ws, 8, None) == 7
    assert lib.lrm_score(C.byref(p), C.byref(X), C.byref(G), None, ws, 1 << 20, None) == 1


def test_select_validation():
    lib = L._lib
    p = _pairs(E=3)
    q_neg = np.array([1, -2, 3], np.int32)
    d = C.c_void_p(0x4000)
    args = (C.byref(p), d, q_neg.ctypes.data, 0, d, d, d, d, 1 << 24, None)
    assert lib.lrm_select(*args) == 6
    assert lib.lrm_select(C.byref(p), d, None, 0, d, d, d, d, 1 << 24, None) == 1
    q = np.array([1, 2, 3], np.int32)
    assert lib.lrm_select(C.byref(p), d, q.ctypes.data, 16, d, d, d, d, 1 << 24, None) == 10
    assert lib.lrm_select(C.byref(p), d, q.ctypes.data, 0, d, d, d, d, 16, None) == 7


def test_grouped_bwd_and_unpermute_validation():
    lib = L._lib
    d = C.c_void_p(0x4000)
    assert lib.lrm_grouped_bwd(0, d, 4, 1, d, d, d, 64 * 64, 64, 64, d, d, d, 1 << 20, None) == 2
    assert lib.lrm_grouped_bwd(4, d, 4, 7, d, d, d, 64 * 64, 64, 64, d, d, d, 1 << 20, None) == 3
    assert lib.lrm_grouped_bwd(4, d, 4, 1, d, d, d, 64 * 64, 60, 64, d, d, d, 1 << 20, None) == 10
    assert lib.lrm_grouped_bwd(4, None, 4, 1, d, d, d, 64 * 64, 64, 64, d, d, d, 1 << 20,
                               None) == 1
    assert lib.lrm_grouped_bwd(4, d, 4, 1, d, d, d, 64 * 64, 64, 64, d, d, d, 4, None) == 7
    # leading dimensions up to 2^20 - 1 (32-bit offsets inside a 256-row tile)
    big = (1 << 20) * 64
    assert lib.lrm_grouped_bwd(4, d, 4, 1, d, d, d, big, 1 << 20, 64, d, d, d, 1 << 20, None) == 2
    assert lib.lrm_grouped_bwd(4, d, 4, 1, d, d, d, big, 64, 1 << 20, d, d, d, 1 << 20, None) == 2
    p = _pairs()
    assert lib.lrm_unpermute(C.byref(p), d, d, 64, 5, d, d, 1 << 20, None) == 4
    assert lib.lrm_unpermute(C.byref(p), d, d, 62, 0, d, d, 1 << 20, None) == 10


def test_expert_backward_validation_and_workspace_size():
    lib = L._lib
    pb = L.lrm_problem()
    pb.kind, pb.dtype = L.LRM_LINEAR, L.LRM_BF16
    pb.pairs = _pairs(T=16, N=32, E=4)
    pb.X = _m(cols=64, ld=64)
    pb.G = _m(rows=L.LRM_ROWS_PAIR, cols=32, ld=32)
    pb.W, pb.w_stride, pb.d_in, pb.d_out = 0x8000, 64 * 32, 64, 32
    q = np.array([4, 0, 9, 100], np.int32)
    pb.quota = q.ctypes.data
    n = lib.lrm_workspace_size(C.byref(pb))
    assert n > 0 and n % 256 == 0
    # packed buffers are sized by min(N, sum q) = 32 rows, not by the quota sum
    q2 = np.array([4, 0, 9, 1000], np.int32)
    pb.quota = q2.ctypes.data
    assert lib.lrm_workspace_size(C.byref(pb)) == n
    # a smaller quota sum shrinks the packed buffers
    q3 = np.array([1, 0, 1, 1], np.int32)
    pb.quota = q3.ctypes.data
    assert lib.lrm_workspace_size(C.byref(pb)) < n
    out = L.lrm_outputs()
    assert lib.lrm_expert_backward(C.byref(pb), C.byref(out), C.c_void_p(0x10000), n, None) == 1
    out.dW, out.dX = 0x9000, 0xA000
    assert lib.lrm_expert_backward(C.byref(pb), C.byref(out), None, n, None) == 7
    assert lib.lrm_expert_backward(C.byref(pb), C.byref(out), C.c_void_p(0x10000), 16, None) == 7
    pb.quota = np.array([1, -1, 1, 1], np.int32).ctypes.data
    assert lib.lrm_workspace_size(C.byref(pb)) == 0
    pb.quota = q.ctypes.data
    # d_in and d_out up to 2^20 - 1
    pb.X = _m(cols=1 << 20, ld=1 << 20)
    pb.d_in, pb.w_stride = 1 << 20, (1 << 20) * 32
    assert lib.lrm_workspace_size(C.byref(pb)) == 0
    pb.X = _m(cols=(1 << 20) - 8, ld=(1 << 20) - 8)  # bf16 rows stay 16-byte aligned
    pb.d_in, pb.w_stride = (1 << 20) - 8, ((1 << 20) - 8) * 32
    assert lib.lrm_workspace_size(C.byref(pb)) > 0
    pb.kind = 5
    assert lib.lrm_workspace_size(C.byref(pb)) == 0


def test_swiglu_workspace_sizes_from_quotas():
    lib = L._lib
    pb = L.lrm_problem()
    pb.kind, pb.dtype = L.LRM_SWIGLU, L.LRM_BF16
    pb.pairs = _pairs(T=64, N=128, E=4)
    pb.X = _m(cols=64, ld=64)
    pb.G = _m(cols=64, ld=64)
    pb.A = _m(rows=L.LRM_ROWS_PAIR, cols=32, ld=32)
    pb.B = _m(rows=L.LRM_ROWS_PAIR, cols=32, ld=32)
    pb.W_gate = pb.W_up = pb.W_down = 0x8000
    pb.H, pb.I = 64, 32
    qd = np.array([8, 8, 8, 8], np.int32)
    qs = np.array([4, 4, 4, 4], np.int32)
    pb.quota_down = pb.quota_gate = pb.quota_up = qd.ctypes.data
    same = lib.lrm_workspace_size(C.byref(pb))
    pb.quota_gate = pb.quota_up = qs.ctypes.data
    second = lib.lrm_workspace_size(C.byref(pb))
    assert same > 0 and second > 0 and same != second
    pb.A = _m(rows=L.LRM_ROWS_TOKEN, cols=32, ld=32)
    assert lib.lrm_workspace_size(C.byref(pb)) == 0
    # H and I up to 2^20 - 1
    pb.A = _m(rows=L.LRM_ROWS_PAIR, cols=1 << 20, ld=1 << 20)
    pb.B = _m(rows=L.LRM_ROWS_PAIR, cols=1 << 20, ld=1 << 20)
    pb.I = 1 << 20
    assert lib.lrm_workspace_size(C.byref(pb)) == 0


def test_receiver_layout_validation_returns_before_launch():
    lib = L._lib
    d = C.c_void_p(0x4000)
    assert lib.lrm_receiver_layout_workspace_size(0, 2) == 0
    assert lib.lrm_receiver_layout_workspace_size(4, 1025) == 0
    n = lib.lrm_receiver_layout_workspace_size(4, 2)
    assert n >= 4 * 3 * 4
    assert lib.lrm_receiver_layout(0, 2, d, d, 8, d, d, d, d, n, None) == 2
    assert lib.lrm_receiver_layout(4, 2, None, d, 8, d, d, d, d, n, None) == 1
    assert lib.lrm_receiver_layout(4, 2, d, d, 8, d, d, None, d, n, None) == 1
    assert lib.lrm_receiver_layout(4, 2, d, d, 8, d, d, d, d, n - 1, None) == 7
    assert lib.lrm_receiver_layout(4, 2, d, d, -1, d, d, d, d, n, None) == 2



def test_quota_on_device_and_debug_flags():
    # LRM_QUOTA_ON_DEVICE: the host never reads the quota arrays (a pointer that
    # is not host memory is fine) and sizes the packed blocks for every pair
    lib = L._lib
    pb = L.lrm_problem()
    pb.kind, pb.dtype = L.LRM_LINEAR, L.LRM_BF16
    pb.pairs = _pairs(T=16, N=32, E=4)
    pb.X = _m(cols=64, ld=64)
    pb.G = _m(rows=L.LRM_ROWS_PAIR, cols=32, ld=32)
    pb.W, pb.w_stride, pb.d_in, pb.d_out = 0x8000, 64 * 32, 64, 32
    q_all = np.array([100, 100, 100, 100], np.int32)
    pb.quota = q_all.ctypes.data
    n_all = lib.lrm_workspace_size(C.byref(pb))
    pb.flags = L.LRM_QUOTA_ON_DEVICE
    pb.quota = 0x10  # a device address: must not be dereferenced on the host
    assert lib.lrm_workspace_size(C.byref(pb)) == n_all
    pb.flags = L.LRM_QUOTA_ON_DEVICE | L.LRM_DEBUG_CHECKS | L.LRM_DW_BF16
    assert lib.lrm_workspace_size(C.byref(pb)) == n_all
    pb.quota = None
    assert lib.lrm_workspace_size(C.byref(pb)) == 0
    pb.quota, pb.flags = 0x10, 32  # not a flag of the ABI
    assert lib.lrm_workspace_size(C.byref(pb)) == 0
    # lrm_select: device quotas must be present; the workspace is still checked
    p = _pairs(E=3)
    d = C.c_void_p(0x4000)
    qdev = L.LRM_QUOTA_ON_DEVICE
    assert lib.lrm_select(C.byref(p), d, None, qdev, d, d, d, d, 1 << 24, None) == 1
    assert lib.lrm_select(C.byref(p), d, C.c_void_p(0x10), qdev, d, d, d, d, 16, None) == 7
