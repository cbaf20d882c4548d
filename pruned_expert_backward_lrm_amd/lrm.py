"""ctypes binding of liblrm.so (the C ABI in include/lrm.h).

Argument marshalling only: every step of the pruned expert backward runs in
the HIP kernels behind the C ABI.  PyTorch provides device memory and the
stream.  Importing this module fails loudly when the library is not built;
there is no fallback implementation.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblrm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -m pruned_expert_backward_lrm_amd.build`")
_lib = C.CDLL(LIB_PATH)

# ------------------------------------------------------------------ constants
LRM_OK = 0
STATUS_NAMES = ["OK", "ERR_NULL", "ERR_SHAPE", "ERR_DTYPE", "ERR_LAYOUT", "ERR_ALIGN",
                "ERR_QUOTA", "ERR_WORKSPACE", "ERR_INDEX", "ERR_HIP", "ERR_UNSUPPORTED",
                "ERR_INFEASIBLE"]
LRM_ERR_INDEX, LRM_ERR_INFEASIBLE = 8, 11
LRM_F32, LRM_BF16 = 0, 1
LRM_ROWS_TOKEN, LRM_ROWS_PAIR = 0, 1
LRM_LINEAR, LRM_SWIGLU = 0, 1
LRM_KEEP_ALL = 1
LRM_DW_BF16 = 2
LRM_QUOTA_ON_DEVICE = 4
LRM_DEBUG_CHECKS = 8
LRM_GATHER_LOADS = 16
ROWS = {"token": LRM_ROWS_TOKEN, "pair": LRM_ROWS_PAIR}


class LrmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.lrm_status_string(status).decode()
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: LRM_{name} ({msg})")


# ------------------------------------------------------------------- structs
class lrm_pairs(C.Structure):
    _fields_ = [("T", C.c_int32), ("N", C.c_int32), ("E", C.c_int32), ("_pad", C.c_int32),
                ("token", C.c_void_p), ("expert", C.c_void_p), ("weight", C.c_void_p)]


class lrm_mat(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("dtype", C.c_int32), ("rows", C.c_int32),
                ("cols", C.c_int32), ("_pad", C.c_int32), ("ld", C.c_int64)]


class lrm_problem(C.Structure):
    _fields_ = [("kind", C.c_int32), ("flags", C.c_uint32), ("dtype", C.c_int32),
                ("_pad", C.c_int32), ("pairs", lrm_pairs), ("X", lrm_mat), ("G", lrm_mat),
                ("W", C.c_void_p), ("w_stride", C.c_int64), ("d_in", C.c_int32),
                ("d_out", C.c_int32), ("quota", C.c_void_p), ("A", lrm_mat), ("B", lrm_mat),
                ("W_gate", C.c_void_p), ("W_up", C.c_void_p), ("W_down", C.c_void_p),
                ("H", C.c_int32), ("I", C.c_int32), ("quota_down", C.c_void_p),
                ("quota_gate", C.c_void_p), ("quota_up", C.c_void_p), ("h_sumsq", C.c_void_p)]


class lrm_outputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "dW", "dW_gate", "dW_up", "dW_down", "dX", "score", "pos", "offsets", "score_gate",
        "score_up", "pos_gate", "pos_up", "offsets_gate", "offsets_up", "dH")]


_P = C.c_void_p
_SZ = C.c_size_t
_I32 = C.c_int32
_sigs = {
    "lrm_status_string": (C.c_char_p, [C.c_int]),
    "lrm_version": (_I32, []),
    "lrm_max_kept": (C.c_int64, [_I32, _I32, _P]),
    "lrm_score": (C.c_int, [C.POINTER(lrm_pairs), C.POINTER(lrm_mat), C.POINTER(lrm_mat), _P,
                            _P, _SZ, _P]),
    "lrm_score_workspace_size": (_SZ, [C.POINTER(lrm_pairs)]),
    "lrm_score_glu": (C.c_int, [C.POINTER(lrm_pairs), C.POINTER(lrm_mat), C.POINTER(lrm_mat),
                                C.POINTER(lrm_mat), _P, _P, _SZ, _P]),
    "lrm_select": (C.c_int, [C.POINTER(lrm_pairs), _P, _P, C.c_uint32, _P, _P, _P, _P, _SZ, _P]),
    "lrm_select_workspace_size": (_SZ, [C.POINTER(lrm_pairs)]),
    "lrm_compact": (C.c_int, [C.POINTER(lrm_pairs), _P, _P, _I32, C.POINTER(lrm_mat),
                              C.POINTER(lrm_mat), _P, _P, _P]),
    "lrm_compact_rows": (C.c_int, [C.POINTER(lrm_pairs), _P, _P, _I32, _P, C.POINTER(lrm_mat),
                                   C.POINTER(lrm_mat), _P, _P, _P]),
    "lrm_grouped_bwd": (C.c_int, [_I32, _P, _I32, _I32, _P, _P, _P, C.c_int64, _I32, _I32, _P, _P,
                                  _P, _SZ, _P]),
    "lrm_grouped_bwd_workspace_size": (_SZ, [_I32]),
    "lrm_unpermute": (C.c_int, [C.POINTER(lrm_pairs), _P, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "lrm_unpermute_workspace_size": (_SZ, [C.POINTER(lrm_pairs)]),
    "lrm_expert_backward": (C.c_int, [C.POINTER(lrm_problem), C.POINTER(lrm_outputs), _P, _SZ,
                                      _P]),
    "lrm_expert_backward_events": (C.c_int, [C.POINTER(lrm_problem), C.POINTER(lrm_outputs), _P,
                                             _SZ, _P, C.POINTER(C.c_void_p), _I32]),
    "lrm_workspace_size": (_SZ, [C.POINTER(lrm_problem)]),
    "lrm_check_device_errors": (C.c_int, [_P, _P]),
    "lrm_select_static": (C.c_int, [C.POINTER(lrm_pairs), _P, _P, C.c_uint32, _P, _P, _P, _P]),
    "lrm_quota_waterfill": (C.c_int, [_I32, _P, C.c_int64, _P]),
    "lrm_quota_waterfill_device": (C.c_int, [C.POINTER(lrm_pairs), _P, C.c_int64, _P, _P, _SZ,
                                             _P]),
    "lrm_quota_waterfill_device_workspace_size": (_SZ, [C.POINTER(lrm_pairs)]),
    "lrm_redistribute": (C.c_int, [_I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ]),
    "lrm_redistribute_workspace_size": (_SZ, [_I32, _I32]),
    "lrm_receiver_layout": (C.c_int, [_I32, _I32, _P, _P, _I32, _P, _P, _P, _P, _SZ, _P]),
    "lrm_receiver_layout_workspace_size": (_SZ, [_I32, _I32]),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sigs)


# ------------------------------------------------------------------- helpers
def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != LRM_OK:
        raise LrmError(status, where)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LRM_BF16
    if t.dtype == torch.float32:
        return LRM_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


class Pairs:
    """The routed pairs of a layer call: device int32 token/expert, fp32 weight."""

    def __init__(self, token: torch.Tensor, expert: torch.Tensor, weight: torch.Tensor,
                 T: int, E: int):
        self.token, self.expert, self.weight = token, expert, weight
        self.T, self.E, self.N = int(T), int(E), int(token.shape[0])
        self.c = lrm_pairs(self.T, self.N, self.E, 0, _ptr(token), _ptr(expert), _ptr(weight))

    @classmethod
    def from_routing(cls, r, device) -> "Pairs":
        return cls(torch.as_tensor(r.token, dtype=torch.int32, device=device),
                   torch.as_tensor(r.expert, dtype=torch.int32, device=device),
                   torch.as_tensor(r.weight, dtype=torch.float32, device=device), r.T, r.E)


def mat(t: torch.Tensor | None, rows: str | int) -> lrm_mat:
    """Describe a row-major device matrix whose rows are addressed via the pairs."""
    if t is None:
        return lrm_mat(None, 0, 0, 0, 0, 0)
    r = ROWS[rows] if isinstance(rows, str) else int(rows)
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("matrices must be 2-D with unit column stride")
    m = lrm_mat(_ptr(t), dtype_code(t), r, t.shape[1], 0, t.stride(0))
    m._tensor = t  # the descriptor keeps its memory alive
    return m


def _ws(nbytes: int, device, ws):
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _quota_arr(q):
    """Quotas as the C ABI takes them: a host int32 array, or (with
    LRM_QUOTA_ON_DEVICE) a contiguous int32 device tensor passed as it is."""
    if isinstance(q, torch.Tensor) and q.is_cuda:
        if q.dtype != torch.int32 or not q.is_contiguous():
            raise ValueError("device quotas must be a contiguous int32 tensor")
        return q
    return np.ascontiguousarray(np.asarray(q, dtype=np.int32))


# ---------------------------------------------------------------- the steps
def lrm_score(pairs: Pairs, X: lrm_mat, G: lrm_mat, score: torch.Tensor, ws=None, stream=None):
    need = _lib.lrm_score_workspace_size(C.byref(pairs.c))
    ws = _ws(need, score.device, ws)
    _check(_lib.lrm_score(C.byref(pairs.c), C.byref(X), C.byref(G), _ptr(score), _ptr(ws),
                          ws.numel(), _stream(stream)), "lrm_score")


def lrm_score_glu(pairs: Pairs, A: lrm_mat, B: lrm_mat, G: lrm_mat, score: torch.Tensor,
                  ws=None, stream=None):
    need = _lib.lrm_score_workspace_size(C.byref(pairs.c))
    ws = _ws(need, score.device, ws)
    _check(_lib.lrm_score_glu(C.byref(pairs.c), C.byref(A), C.byref(B), C.byref(G),
                              _ptr(score), _ptr(ws), ws.numel(), _stream(stream)),
           "lrm_score_glu")


def lrm_select(pairs: Pairs, score, quota, pos, offsets, kept, flags=0, ws=None, stream=None,
               device=None):
    need = _lib.lrm_select_workspace_size(C.byref(pairs.c))
    ws = _ws(need, device or offsets.device, ws)
    q = _quota_arr(quota) if quota is not None else None
    _check(_lib.lrm_select(C.byref(pairs.c), _ptr(score), _ptr(q), flags, _ptr(pos),
                           _ptr(offsets), _ptr(kept), _ptr(ws), ws.numel(), _stream(stream)),
           "lrm_select")
    return ws


def lrm_select_static(pairs: Pairs, score, quota, pos, offsets, kept, flags=0, stream=None):
    """lrm_select with the library's own scratch array (no workspace, no
    allocation)."""
    q = _quota_arr(quota) if quota is not None else None
    _check(_lib.lrm_select_static(C.byref(pairs.c), _ptr(score), _ptr(q), flags, _ptr(pos),
                                  _ptr(offsets), _ptr(kept), _stream(stream)),
           "lrm_select_static")


def lrm_compact(pairs: Pairs, kept, offsets, max_rows: int, X: lrm_mat, G: lrm_mat, Xp, Gp,
                stream=None):
    _check(_lib.lrm_compact(C.byref(pairs.c), _ptr(kept), _ptr(offsets), int(max_rows),
                            C.byref(X), C.byref(G), _ptr(Xp), _ptr(Gp), _stream(stream)),
           "lrm_compact")


def lrm_compact_rows(pairs: Pairs, kept, offsets, max_rows: int, dst, X: lrm_mat, G: lrm_mat,
                     Xp, Gp, stream=None):
    """lrm_compact writing packed row m to row dst[m] (receiver-major rows)."""
    _check(_lib.lrm_compact_rows(C.byref(pairs.c), _ptr(kept), _ptr(offsets), int(max_rows),
                                 _ptr(dst), C.byref(X), C.byref(G), _ptr(Xp), _ptr(Gp),
                                 _stream(stream)),
           "lrm_compact_rows")


def lrm_grouped_bwd(E: int, offsets, max_rows: int, Gp, Xp, W, d_in: int, d_out: int, dW, dXp,
                    dtype=None, w_stride=None, ws=None, stream=None):
    dt = dtype if dtype is not None else dtype_code(Gp)
    if w_stride is None:
        w_stride = d_in * d_out
    need = _lib.lrm_grouped_bwd_workspace_size(int(E))
    ws = _ws(need, offsets.device, ws)
    _check(_lib.lrm_grouped_bwd(int(E), _ptr(offsets), int(max_rows), dt, _ptr(Gp), _ptr(Xp),
                                _ptr(W), int(w_stride), int(d_in), int(d_out), _ptr(dW),
                                _ptr(dXp), _ptr(ws), ws.numel(), _stream(stream)),
           "lrm_grouped_bwd")


def lrm_unpermute(pairs: Pairs, pos, dXp, d_in: int, out_rows, dX, ws=None, stream=None):
    need = _lib.lrm_unpermute_workspace_size(C.byref(pairs.c))
    ws = _ws(need, dX.device, ws)
    r = ROWS[out_rows] if isinstance(out_rows, str) else int(out_rows)
    _check(_lib.lrm_unpermute(C.byref(pairs.c), _ptr(pos), _ptr(dXp), int(d_in), r, _ptr(dX),
                              _ptr(ws), ws.numel(), _stream(stream)), "lrm_unpermute")


def lrm_max_kept(N: int, quota) -> int:
    q = _quota_arr(quota)
    return int(_lib.lrm_max_kept(int(N), int(q.shape[0]), q.ctypes.data))


def lrm_quota_waterfill(counts, budget: int) -> np.ndarray:
    """Host call: water-filling quotas [E] for candidate counts [E] under a
    pair budget."""
    n = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    q = np.zeros_like(n)
    _check(_lib.lrm_quota_waterfill(int(n.shape[0]), _ptr(n), int(budget), _ptr(q)),
           "lrm_quota_waterfill")
    return q


def lrm_quota_waterfill_device(pairs: Pairs, budget: int, quota, counts=None, ws=None,
                               stream=None):
    """Device call: water-filling quotas written to the device int32 [E] tensor
    `quota`, from device counts [E] or (counts None) the pairs' own counts.
    Returns the workspace (its error word reports pairs out of range)."""
    need = _lib.lrm_quota_waterfill_device_workspace_size(C.byref(pairs.c))
    ws = _ws(need, quota.device, ws)
    _check(_lib.lrm_quota_waterfill_device(C.byref(pairs.c), _ptr(counts), int(budget),
                                           _ptr(quota), _ptr(ws), ws.numel(), _stream(stream)),
           "lrm_quota_waterfill_device")
    return ws


def lrm_redistribute(kept, replica, base=None, cap=None):
    """Host call: the peak-minimising integer assignment of each expert's kept
    pairs to its replicas.  kept [E], replica [E][G] (bool), base/cap [G] or
    None.  Returns (peak, assign int32 [E][G]) as NumPy."""
    k = np.ascontiguousarray(np.asarray(kept, dtype=np.int32))
    rep = np.ascontiguousarray(np.asarray(replica).astype(np.uint8))
    E, G = rep.shape
    b = None if base is None else np.ascontiguousarray(np.asarray(base, dtype=np.int64))
    c = None if cap is None else np.ascontiguousarray(np.asarray(cap, dtype=np.int64))
    assign = np.zeros((E, G), np.int32)
    peak = np.zeros(1, np.int64)
    ws = np.empty(max(int(_lib.lrm_redistribute_workspace_size(E, G)), 64), np.uint8)
    _check(_lib.lrm_redistribute(E, G, _ptr(k), _ptr(rep), _ptr(b), _ptr(c), _ptr(assign),
                                 _ptr(peak), _ptr(ws), ws.nbytes), "lrm_redistribute")
    return int(peak[0]), assign


def lrm_receiver_layout(offsets, assign, max_rows: int, ws=None, stream=None):
    """Device call: receiver-major layout of the packed rows for a device
    assignment [E][G].  Returns (send_off [G+1], blk_off [G][E+1], dst
    [max_rows], ws) device int32 tensors."""
    E, G = int(assign.shape[0]), int(assign.shape[1])
    dev = offsets.device
    i32 = dict(dtype=torch.int32, device=dev)
    send_off = torch.empty(G + 1, **i32)
    blk_off = torch.empty(G, E + 1, **i32)
    dst = torch.empty(max(int(max_rows), 1), **i32)
    ws = _ws(_lib.lrm_receiver_layout_workspace_size(E, G), dev, ws)
    _check(_lib.lrm_receiver_layout(E, G, _ptr(offsets), _ptr(assign), int(max_rows),
                                    _ptr(send_off), _ptr(blk_off), _ptr(dst), _ptr(ws),
                                    ws.numel(), _stream(stream)), "lrm_receiver_layout")
    return send_off, blk_off, dst, ws


def lrm_check_device_errors(ws, stream=None) -> int:
    return int(_lib.lrm_check_device_errors(_ptr(ws), _stream(stream)))


# ---------------------------------------------------------- the fused call
class Problem:
    """An lrm_problem plus the objects that keep its memory alive."""

    def __init__(self, kind: int, pairs: Pairs, dtype: int, flags: int = 0):
        self.keep = [pairs]
        self.c = lrm_problem()
        self.c.kind, self.c.flags, self.c.dtype = kind, flags, dtype
        self.c.pairs = pairs.c
        self.pairs = pairs

    def hold(self, *objs):
        self.keep.extend(objs)


def linear_problem(pairs: Pairs, X, x_rows, G, g_rows, W, quota, flags=0) -> Problem:
    pb = Problem(LRM_LINEAR, pairs, dtype_code(X), flags)
    q = _quota_arr(quota) if quota is not None else None
    pb.hold(X, G, W, q)
    c = pb.c
    c.X, c.G = mat(X, x_rows), mat(G, g_rows)
    c.W, c.w_stride = _ptr(W), W.stride(0)
    c.d_in, c.d_out = X.shape[1], G.shape[1]
    c.quota = _ptr(q)
    return pb


def swiglu_problem(pairs: Pairs, X, x_rows, G, g_rows, A, B, W_gate, W_up, W_down,
                   quota_down, quota_gate, quota_up, flags=0, h_sumsq=None) -> Problem:
    pb = Problem(LRM_SWIGLU, pairs, dtype_code(X), flags)
    qs = [(_quota_arr(q) if q is not None else None) for q in (quota_down, quota_gate, quota_up)]
    pb.hold(X, G, A, B, W_gate, W_up, W_down, *qs, h_sumsq)
    pb.c.h_sumsq = _ptr(h_sumsq)
    c = pb.c
    c.X, c.G = mat(X, x_rows), mat(G, g_rows)
    c.A, c.B = mat(A, "pair"), mat(B, "pair")
    c.W_gate, c.W_up, c.W_down = _ptr(W_gate), _ptr(W_up), _ptr(W_down)
    c.H, c.I = X.shape[1], A.shape[1]
    c.quota_down, c.quota_gate, c.quota_up = (_ptr(q) for q in qs)
    return pb


def lrm_workspace_size(pb: Problem) -> int:
    return int(_lib.lrm_workspace_size(C.byref(pb.c)))


def _outputs(outputs: dict) -> lrm_outputs:
    o = lrm_outputs()
    for k, v in outputs.items():
        setattr(o, k, _ptr(v))
    return o


def _fused_ws(pb: Problem, ws):
    if ws is not None:
        return ws
    n = lrm_workspace_size(pb)
    if n == 0:
        raise LrmError(2, "lrm_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=pb.pairs.token.device)


def lrm_expert_backward(pb: Problem, outputs: dict, ws=None, stream=None):
    o = _outputs(outputs)
    ws = _fused_ws(pb, ws)
    _check(_lib.lrm_expert_backward(C.byref(pb.c), C.byref(o), _ptr(ws), ws.numel(),
                                    _stream(stream)), "lrm_expert_backward")
    return ws


def lrm_expert_backward_events(pb: Problem, outputs: dict, events, ws=None, stream=None):
    """The fused call recording torch.cuda.Event objects at stage boundaries
    (each event must have been recorded once so that its handle exists)."""
    o = _outputs(outputs)
    ws = _fused_ws(pb, ws)
    arr = (C.c_void_p * len(events))(*[ev.cuda_event for ev in events])
    _check(_lib.lrm_expert_backward_events(C.byref(pb.c), C.byref(o), _ptr(ws), ws.numel(),
                                           _stream(stream), arr, len(events)),
           "lrm_expert_backward_events")
    return ws
