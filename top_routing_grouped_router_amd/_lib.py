"""ctypes binding of libmoe.so (the C ABI in include/moe.h).

Argument marshalling only: every function here checks tensor placement and
dtypes, turns torch tensors into device pointers, passes torch's current HIP
stream, and raises MoEError when the library returns a non-zero status.  All
computation happens in the library's HIP kernels.  There is no fallback: if
the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_F32 = 0
MOE_BF16 = 1

STATUS_NAMES = {
    0: "MOE_OK",
    1: "MOE_ERR_INVALID_ARGUMENT",
    2: "MOE_ERR_UNSUPPORTED",
    3: "MOE_ERR_WORKSPACE",
    4: "MOE_ERR_INVALID_PLACEMENT",
    5: "MOE_ERR_HIP",
}

EXPORTED = (
    "moe_status_string", "moe_last_error", "moe_workspace_bytes", "moe_route", "moe_permute",
    "moe_grouped_swiglu_fwd", "moe_combine", "moe_combine_bwd", "moe_grouped_swiglu_bwd",
    "moe_route_bwd", "moe_coselect", "moe_dispatch_plan", "moe_placement_greedy",
    "moe_check_placement", "moe_expert_up", "moe_expert_down", "moe_expert_dgrad_down",
    "moe_expert_dgrad_up", "moe_expert_wgrad", "moe_expert_wgrad_launches",
    "moe_grouped_swiglu_bwd_workspace_bytes",
    "moe_grouped_swiglu_fwd_gather", "moe_grouped_swiglu_bwd_gather", "moe_expert_up_gather",
    "moe_expert_wgrad_gather", "moe_dispatch_pack", "moe_dispatch_expand",
    "moe_expert_capacity", "moe_capacity", "moe_router_zloss", "moe_route_bwd_dense",
    "moe_coselect_cross", "moe_shuffle_plan", "moe_route_flips",
    "moe_gate_folded_supported", "moe_dgate_parts", "moe_permute_gates",
    "moe_expert_up_folded", "moe_expert_dgrad_down_folded", "moe_dgate_from_parts",
    "moe_expert_wgrad_folded", "moe_route_bwd_folded", "moe_route_noalloc",
    "moe_route_noalloc_max_bytes",
)


class MoEError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, f"status {status}")
        super().__init__(f"{func}: {self.name}: {detail}")


class moe_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("f", ctypes.c_int32), ("k", ctypes.c_int32), ("act", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
_DIMS = ctypes.POINTER(moe_dims)

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_bytes": (_SZ, [_DIMS, _I32]),
    "moe_expert_wgrad_launches": (_I32, [_DIMS]),
    "moe_route": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _F32, _P, _I32, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_noalloc": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _F32, _P, _I32, _P, _P, _P, _P]),
    "moe_route_noalloc_max_bytes": (_SZ, []),
    "moe_permute": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_swiglu_fwd": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_combine": (_I32, [_DIMS, _P, _P, _P, _P, _P]),
    "moe_combine_bwd": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_swiglu_bwd": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _I32, _P, _SZ, _P]),
    "moe_grouped_swiglu_bwd_workspace_bytes": (_SZ, [_DIMS, _I32]),
    "moe_route_bwd": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_coselect": (_I32, [_I64, _I32, _I32, _P, _P, _P]),
    "moe_dispatch_plan": (_I32, [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _SZ, _P]),
    "moe_placement_greedy": (_I32, [_I32, _I32, _P, _P]),
    "moe_expert_up": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_down": (_I32, [_DIMS, _P, _P, _P, _P, _P]),
    "moe_expert_dgrad_down": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_dgrad_up": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_wgrad": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _SZ, _P]),
    "moe_expert_up_gather": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_pack": (_I32, [_DIMS, _I32, _P, _P, _P, _P, _P]),
    "moe_dispatch_expand": (_I32, [_DIMS, _P, _P, _P, _P, _P]),
    "moe_expert_wgrad_gather": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                                       _SZ, _P]),
    "moe_grouped_swiglu_fwd_gather": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _SZ, _P]),
    "moe_grouped_swiglu_bwd_gather": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _I32, _P, _SZ, _P]),
    "moe_check_placement": (_I32, [_I32, _I32, _P]),
    "moe_expert_capacity": (_I32, [_I64, _I32, _I32, _I32, ctypes.c_double]),
    "moe_gate_folded_supported": (_I32, [_DIMS]),
    "moe_dgate_parts": (_I32, [_DIMS]),
    "moe_permute_gates": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_up_folded": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_dgrad_down_folded": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P]),
    "moe_dgate_from_parts": (_I32, [_DIMS, _P, _P, _P, _P]),
    "moe_route_bwd_folded": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _SZ, _P]),
    "moe_expert_wgrad_folded": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_capacity": (_I32, [_DIMS, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "moe_router_zloss": (_I32, [_DIMS, _P, _I32, _P, _P, _SZ, _P]),
    "moe_route_bwd_dense": (_I32, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _F32, _F32,
                                   _P, _P, _P, _P, _SZ, _P]),
    "moe_coselect_cross": (_I32, [_I64, _I32, _I32, _P, _P, _P, _P]),
    "moe_route_flips": (_I32, [_I64, _I32, _I32, _P, _P, _P, _P, _P]),
    "moe_shuffle_plan": (_I32, [_I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                _P]),
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m top_routing_grouped_router_amd.build` (no CPU fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(status: int, func: str) -> None:
    if status != 0:
        raise MoEError(status, func, last_error())


def make_dims(T: int, d: int, E: int, f: int, k: int, act) -> moe_dims:
    if isinstance(act, torch.dtype):
        act = MOE_BF16 if act == torch.bfloat16 else MOE_F32
    return moe_dims(int(T), int(d), int(E), int(f), int(k), int(act))


def act_dtype(dims: moe_dims) -> torch.dtype:
    return torch.bfloat16 if dims.act == MOE_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def workspace_bytes(dims: moe_dims, n_groups: int = 1) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(dims), int(n_groups)))


def alloc_workspace(dims: moe_dims, n_groups: int = 1, device="cuda") -> torch.Tensor:
    n = max(workspace_bytes(dims, n_groups), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def moe_route(dims, x, w_router, logits, topk_idx, topk_gate, margin, near_tie_eps,
              near_tie_count, n_groups, group_count, group_mean_prob, group_aux, workspace,
              stream=None):
    act = act_dtype(dims)
    st = lib().moe_route(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(w_router, "w_router", torch.float32),
        _ptr(logits, "logits", torch.float32), _ptr(topk_idx, "topk_idx", torch.int32),
        _ptr(topk_gate, "topk_gate", torch.float32), _ptr(margin, "margin", torch.float32),
        float(near_tie_eps), _ptr(near_tie_count, "near_tie_count", torch.int32), int(n_groups),
        _ptr(group_count, "group_count", torch.int32),
        _ptr(group_mean_prob, "group_mean_prob", torch.float32),
        _ptr(group_aux, "group_aux", torch.float32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_route")


def moe_route_noalloc(dims, x, w_router, logits, topk_idx, topk_gate, margin, near_tie_eps,
                      near_tie_count, n_groups, group_count, group_mean_prob, group_aux,
                      stream=None):
    act = act_dtype(dims)
    st = lib().moe_route_noalloc(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(w_router, "w_router", torch.float32),
        _ptr(logits, "logits", torch.float32), _ptr(topk_idx, "topk_idx", torch.int32),
        _ptr(topk_gate, "topk_gate", torch.float32), _ptr(margin, "margin", torch.float32),
        float(near_tie_eps), _ptr(near_tie_count, "near_tie_count", torch.int32), int(n_groups),
        _ptr(group_count, "group_count", torch.int32),
        _ptr(group_mean_prob, "group_mean_prob", torch.float32),
        _ptr(group_aux, "group_aux", torch.float32), _stream(stream))
    _check(st, "moe_route_noalloc")


def moe_route_noalloc_max_bytes() -> int:
    return int(lib().moe_route_noalloc_max_bytes())


def moe_permute(dims, topk_idx, expert_counts, expert_offsets, pos, src_token, x, x_perm,
                workspace, stream=None):
    act = act_dtype(dims)
    st = lib().moe_permute(
        ctypes.byref(dims), _ptr(topk_idx, "topk_idx", torch.int32),
        _ptr(expert_counts, "expert_counts", torch.int32),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(pos, "pos", torch.int32),
        _ptr(src_token, "src_token", torch.int32), _ptr(x, "x", act), _ptr(x_perm, "x_perm", act),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "moe_permute")


def moe_grouped_swiglu_fwd(dims, x_perm, expert_offsets, w1, w3, w2, a_save, b_save, h_save,
                           y_perm, workspace=None, stream=None):
    act = act_dtype(dims)
    st = lib().moe_grouped_swiglu_fwd(
        ctypes.byref(dims), _ptr(x_perm, "x_perm", act),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(w1, "w1", act),
        _ptr(w3, "w3", act), _ptr(w2, "w2", act), _ptr(a_save, "a_save", act),
        _ptr(b_save, "b_save", act), _ptr(h_save, "h_save", act), _ptr(y_perm, "y_perm", act),
        _ptr(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "moe_grouped_swiglu_fwd")


def moe_combine(dims, rows, pos, gate, out, stream=None):
    act = act_dtype(dims)
    st = lib().moe_combine(ctypes.byref(dims), _ptr(rows, "rows", act),
                           _ptr(pos, "pos", torch.int32), _ptr(gate, "gate", torch.float32),
                           _ptr(out, "out", act), _stream(stream))
    _check(st, "moe_combine")


def moe_combine_bwd(dims, dy, y_perm, pos, gate, dy_perm, dgate, stream=None):
    act = act_dtype(dims)
    st = lib().moe_combine_bwd(ctypes.byref(dims), _ptr(dy, "dy", act),
                               _ptr(y_perm, "y_perm", act), _ptr(pos, "pos", torch.int32),
                               _ptr(gate, "gate", torch.float32), _ptr(dy_perm, "dy_perm", act),
                               _ptr(dgate, "dgate", torch.float32), _stream(stream))
    _check(st, "moe_combine_bwd")


def _wgrad_dtype(dims, wgrad_dtype):
    """(moe_dtype code, torch dtype) of the weight gradients; None: the act type."""
    if wgrad_dtype is None:
        wgrad_dtype = int(dims.act)
    if wgrad_dtype in (torch.float32, MOE_F32):
        return MOE_F32, torch.float32
    if wgrad_dtype in (torch.bfloat16, MOE_BF16):
        return MOE_BF16, torch.bfloat16
    raise ValueError(f"wgrad_dtype must be MOE_F32 or MOE_BF16, got {wgrad_dtype!r}")


def moe_grouped_swiglu_bwd_workspace_bytes(dims, recompute: bool) -> int:
    return int(lib().moe_grouped_swiglu_bwd_workspace_bytes(ctypes.byref(dims), int(bool(recompute))))


def moe_grouped_swiglu_bwd(dims, x_perm, expert_offsets, w1, w3, w2, a_save, b_save, h_save,
                           dy_perm, dx_perm, dw1, dw3, dw2, workspace, stream=None,
                           wgrad_dtype=None):
    act = act_dtype(dims)
    wcode, wdt = _wgrad_dtype(dims, wgrad_dtype)
    st = lib().moe_grouped_swiglu_bwd(
        ctypes.byref(dims), _ptr(x_perm, "x_perm", act),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(w1, "w1", act),
        _ptr(w3, "w3", act), _ptr(w2, "w2", act), _ptr(a_save, "a_save", act),
        _ptr(b_save, "b_save", act), _ptr(h_save, "h_save", act), _ptr(dy_perm, "dy_perm", act),
        _ptr(dx_perm, "dx_perm", act), _ptr(dw1, "dw1", wdt), _ptr(dw3, "dw3", wdt),
        _ptr(dw2, "dw2", wdt), wcode, _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_grouped_swiglu_bwd")


def moe_route_bwd(dims, x, w_router, topk_idx, topk_gate, dgate, expert_offsets, pos, src_token,
                  dx_perm, dx, dw_router, workspace, stream=None):
    act = act_dtype(dims)
    st = lib().moe_route_bwd(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(w_router, "w_router", torch.float32),
        _ptr(topk_idx, "topk_idx", torch.int32), _ptr(topk_gate, "topk_gate", torch.float32),
        _ptr(dgate, "dgate", torch.float32), _ptr(expert_offsets, "expert_offsets", torch.int32),
        _ptr(pos, "pos", torch.int32), _ptr(src_token, "src_token", torch.int32),
        _ptr(dx_perm, "dx_perm", act), _ptr(dx, "dx", act),
        _ptr(dw_router, "dw_router", torch.float32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_route_bwd")


def moe_expert_up(dims, x_perm, expert_offsets, w1, w3, a_save, b_save, h_save, stream=None):
    act = act_dtype(dims)
    st = lib().moe_expert_up(ctypes.byref(dims), _ptr(x_perm, "x_perm", act),
                             _ptr(expert_offsets, "expert_offsets", torch.int32),
                             _ptr(w1, "w1", act), _ptr(w3, "w3", act),
                             _ptr(a_save, "a_save", act), _ptr(b_save, "b_save", act),
                             _ptr(h_save, "h_save", act), _stream(stream))
    _check(st, "moe_expert_up")


def moe_expert_down(dims, h_save, expert_offsets, w2, y_perm, stream=None):
    act = act_dtype(dims)
    st = lib().moe_expert_down(ctypes.byref(dims), _ptr(h_save, "h_save", act),
                               _ptr(expert_offsets, "expert_offsets", torch.int32),
                               _ptr(w2, "w2", act), _ptr(y_perm, "y_perm", act), _stream(stream))
    _check(st, "moe_expert_down")


def moe_expert_dgrad_down(dims, dy_perm, expert_offsets, w2, a_save, b_save, da, db,
                          stream=None):
    act = act_dtype(dims)
    st = lib().moe_expert_dgrad_down(ctypes.byref(dims), _ptr(dy_perm, "dy_perm", act),
                                     _ptr(expert_offsets, "expert_offsets", torch.int32),
                                     _ptr(w2, "w2", act), _ptr(a_save, "a_save", act),
                                     _ptr(b_save, "b_save", act), _ptr(da, "da", act),
                                     _ptr(db, "db", act), _stream(stream))
    _check(st, "moe_expert_dgrad_down")


def moe_expert_dgrad_up(dims, da, db, expert_offsets, w1, w3, dx_perm, stream=None):
    act = act_dtype(dims)
    st = lib().moe_expert_dgrad_up(ctypes.byref(dims), _ptr(da, "da", act), _ptr(db, "db", act),
                                   _ptr(expert_offsets, "expert_offsets", torch.int32),
                                   _ptr(w1, "w1", act), _ptr(w3, "w3", act),
                                   _ptr(dx_perm, "dx_perm", act), _stream(stream))
    _check(st, "moe_expert_dgrad_up")


def moe_expert_wgrad(dims, x_perm, expert_offsets, h_save, dy_perm, da, db, dw1, dw3, dw2,
                     workspace, stream=None, wgrad_dtype=None):
    act = act_dtype(dims)
    wcode, wdt = _wgrad_dtype(dims, wgrad_dtype)
    st = lib().moe_expert_wgrad(
        ctypes.byref(dims), _ptr(x_perm, "x_perm", act),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(h_save, "h_save", act),
        _ptr(dy_perm, "dy_perm", act), _ptr(da, "da", act), _ptr(db, "db", act),
        _ptr(dw1, "dw1", wdt), _ptr(dw3, "dw3", wdt), _ptr(dw2, "dw2", wdt), wcode,
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "moe_expert_wgrad")


def moe_coselect(T, k, E, topk_idx, coselect, stream=None):
    st = lib().moe_coselect(int(T), int(k), int(E), _ptr(topk_idx, "topk_idx", torch.int32),
                            _ptr(coselect, "coselect", torch.int32), _stream(stream))
    _check(st, "moe_coselect")


def moe_dispatch_plan(T, k, E, G, topk_idx, placement, n_dest, group_rows, group_offsets,
                      row_token, assign_row, stats, workspace, stream=None):
    pl = (ctypes.c_int32 * E)(*[int(v) for v in placement])
    st = lib().moe_dispatch_plan(
        int(T), int(k), int(E), int(G), _ptr(topk_idx, "topk_idx", torch.int32),
        ctypes.cast(pl, ctypes.c_void_p), _ptr(n_dest, "n_dest", torch.int32),
        _ptr(group_rows, "group_rows", torch.int32),
        _ptr(group_offsets, "group_offsets", torch.int32),
        _ptr(row_token, "row_token", torch.int32), _ptr(assign_row, "assign_row", torch.int32),
        _ptr(stats, "stats", torch.int32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_dispatch_plan")


def moe_placement_greedy(E, G, coselect) -> list:
    import numpy as np
    W = np.ascontiguousarray(np.asarray(coselect, dtype=np.int64))
    if W.shape != (E, E):
        raise ValueError("coselect must be [E, E]")
    out = (ctypes.c_int32 * E)()
    st = lib().moe_placement_greedy(int(E), int(G), W.ctypes.data_as(ctypes.c_void_p),
                                    ctypes.cast(out, ctypes.c_void_p))
    _check(st, "moe_placement_greedy")
    return list(out)


def moe_check_placement(E, G, placement) -> None:
    pl = (ctypes.c_int32 * E)(*[int(v) for v in placement])
    st = lib().moe_check_placement(int(E), int(G), ctypes.cast(pl, ctypes.c_void_p))
    _check(st, "moe_check_placement")


# ---------------------------------------------------------------- gathered expert input
def moe_grouped_swiglu_fwd_gather(dims, x, src_token, expert_offsets, w1, w3, w2, a_save,
                                  b_save, h_save, y_perm, workspace=None, stream=None):
    act = act_dtype(dims)
    st = lib().moe_grouped_swiglu_fwd_gather(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(src_token, "src_token", torch.int32),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(w1, "w1", act),
        _ptr(w3, "w3", act), _ptr(w2, "w2", act), _ptr(a_save, "a_save", act),
        _ptr(b_save, "b_save", act), _ptr(h_save, "h_save", act), _ptr(y_perm, "y_perm", act),
        _ptr(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "moe_grouped_swiglu_fwd_gather")


def moe_grouped_swiglu_bwd_gather(dims, x, src_token, expert_offsets, w1, w3, w2, a_save,
                                  b_save, h_save, dy_perm, dx_perm, dw1, dw3, dw2, workspace,
                                  stream=None, wgrad_dtype=None):
    act = act_dtype(dims)
    wcode, wdt = _wgrad_dtype(dims, wgrad_dtype)
    st = lib().moe_grouped_swiglu_bwd_gather(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(src_token, "src_token", torch.int32),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(w1, "w1", act),
        _ptr(w3, "w3", act), _ptr(w2, "w2", act), _ptr(a_save, "a_save", act),
        _ptr(b_save, "b_save", act), _ptr(h_save, "h_save", act), _ptr(dy_perm, "dy_perm", act),
        _ptr(dx_perm, "dx_perm", act), _ptr(dw1, "dw1", wdt), _ptr(dw3, "dw3", wdt),
        _ptr(dw2, "dw2", wdt), wcode, _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_grouped_swiglu_bwd_gather")


def moe_expert_up_gather(dims, x, src_token, expert_offsets, w1, w3, a_save, b_save, h_save,
                         stream=None):
    act = act_dtype(dims)
    st = lib().moe_expert_up_gather(ctypes.byref(dims), _ptr(x, "x", act),
                                    _ptr(src_token, "src_token", torch.int32),
                                    _ptr(expert_offsets, "expert_offsets", torch.int32),
                                    _ptr(w1, "w1", act), _ptr(w3, "w3", act),
                                    _ptr(a_save, "a_save", act), _ptr(b_save, "b_save", act),
                                    _ptr(h_save, "h_save", act), _stream(stream))
    _check(st, "moe_expert_up_gather")


def moe_expert_wgrad_gather(dims, x, src_token, expert_offsets, h_save, dy_perm, da, db, dw1,
                            dw3, dw2, workspace, stream=None, wgrad_dtype=None):
    act = act_dtype(dims)
    wcode, wdt = _wgrad_dtype(dims, wgrad_dtype)
    st = lib().moe_expert_wgrad_gather(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(src_token, "src_token", torch.int32),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(h_save, "h_save", act),
        _ptr(dy_perm, "dy_perm", act), _ptr(da, "da", act), _ptr(db, "db", act),
        _ptr(dw1, "dw1", wdt), _ptr(dw3, "dw3", wdt), _ptr(dw2, "dw2", wdt), wcode,
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "moe_expert_wgrad_gather")


# ------------------------------------------------- gate folded into the expert rows
def moe_gate_folded_supported(dims) -> bool:
    return bool(lib().moe_gate_folded_supported(ctypes.byref(dims)))


def moe_dgate_parts(dims) -> int:
    return int(lib().moe_dgate_parts(ctypes.byref(dims)))


def moe_permute_gates(dims, topk_idx, topk_gate, expert_counts, expert_offsets, pos, src_token,
                      gate_perm, workspace, stream=None):
    st = lib().moe_permute_gates(
        ctypes.byref(dims), _ptr(topk_idx, "topk_idx", torch.int32),
        _ptr(topk_gate, "topk_gate", torch.float32),
        _ptr(expert_counts, "expert_counts", torch.int32),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(pos, "pos", torch.int32),
        _ptr(src_token, "src_token", torch.int32), _ptr(gate_perm, "gate_perm", torch.float32),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "moe_permute_gates")


def moe_expert_up_folded(dims, x, src_token, expert_offsets, gate_perm, w1, w3, a_save, b_save,
                         hg_save, stream=None):
    act = act_dtype(dims)
    st = lib().moe_expert_up_folded(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(src_token, "src_token", torch.int32),
        _ptr(expert_offsets, "expert_offsets", torch.int32),
        _ptr(gate_perm, "gate_perm", torch.float32), _ptr(w1, "w1", act), _ptr(w3, "w3", act),
        _ptr(a_save, "a_save", act), _ptr(b_save, "b_save", act), _ptr(hg_save, "hg_save", act),
        _stream(stream))
    _check(st, "moe_expert_up_folded")


def moe_expert_dgrad_down_folded(dims, dy, src_token, expert_offsets, gate_perm, w2, a_save,
                                 b_save, da, db, dgate_part, stream=None):
    act = act_dtype(dims)
    st = lib().moe_expert_dgrad_down_folded(
        ctypes.byref(dims), _ptr(dy, "dy", act), _ptr(src_token, "src_token", torch.int32),
        _ptr(expert_offsets, "expert_offsets", torch.int32),
        _ptr(gate_perm, "gate_perm", torch.float32), _ptr(w2, "w2", act),
        _ptr(a_save, "a_save", act), _ptr(b_save, "b_save", act), _ptr(da, "da", act),
        _ptr(db, "db", act), _ptr(dgate_part, "dgate_part", torch.float32), _stream(stream))
    _check(st, "moe_expert_dgrad_down_folded")


def moe_dgate_from_parts(dims, dgate_part, pos, dgate, stream=None):
    st = lib().moe_dgate_from_parts(
        ctypes.byref(dims), _ptr(dgate_part, "dgate_part", torch.float32),
        _ptr(pos, "pos", torch.int32), _ptr(dgate, "dgate", torch.float32), _stream(stream))
    _check(st, "moe_dgate_from_parts")


def moe_expert_wgrad_folded(dims, x, dy, src_token, expert_offsets, hg_save, da, db, dw1, dw3,
                            dw2, stream=None):
    act = act_dtype(dims)
    st = lib().moe_expert_wgrad_folded(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(dy, "dy", act),
        _ptr(src_token, "src_token", torch.int32),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(hg_save, "hg_save", act),
        _ptr(da, "da", act), _ptr(db, "db", act), _ptr(dw1, "dw1", act), _ptr(dw3, "dw3", act),
        _ptr(dw2, "dw2", act), _stream(stream))
    _check(st, "moe_expert_wgrad_folded")


def moe_route_bwd_folded(dims, x, w_router, topk_idx, topk_gate, dgate_part, expert_offsets,
                         pos, src_token, dx_perm, dgate, dx, dw_router, workspace, stream=None):
    act = act_dtype(dims)
    st = lib().moe_route_bwd_folded(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(w_router, "w_router", torch.float32),
        _ptr(topk_idx, "topk_idx", torch.int32), _ptr(topk_gate, "topk_gate", torch.float32),
        _ptr(dgate_part, "dgate_part", torch.float32),
        _ptr(expert_offsets, "expert_offsets", torch.int32), _ptr(pos, "pos", torch.int32),
        _ptr(src_token, "src_token", torch.int32), _ptr(dx_perm, "dx_perm", act),
        _ptr(dgate, "dgate", torch.float32), _ptr(dx, "dx", act),
        _ptr(dw_router, "dw_router", torch.float32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_route_bwd_folded")


# ---------------------------------------------------------------- EP dispatch on one device
def moe_dispatch_pack(dims, G, x, group_offsets, row_token, send, stream=None):
    act = act_dtype(dims)
    st = lib().moe_dispatch_pack(ctypes.byref(dims), int(G), _ptr(x, "x", act),
                                 _ptr(group_offsets, "group_offsets", torch.int32),
                                 _ptr(row_token, "row_token", torch.int32),
                                 _ptr(send, "send", act), _stream(stream))
    _check(st, "moe_dispatch_pack")


def moe_dispatch_expand(dims, recv, assign_row, pos, x_perm, stream=None):
    act = act_dtype(dims)
    st = lib().moe_dispatch_expand(ctypes.byref(dims), _ptr(recv, "recv", act),
                                   _ptr(assign_row, "assign_row", torch.int32),
                                   _ptr(pos, "pos", torch.int32), _ptr(x_perm, "x_perm", act),
                                   _stream(stream))
    _check(st, "moe_dispatch_expand")


# ---------------------------------------------------------------- definitional variants
def moe_expert_capacity(T, k, E, n_groups, factor) -> int:
    c = int(lib().moe_expert_capacity(int(T), int(k), int(E), int(n_groups), float(factor)))
    if c < 0:
        raise MoEError(1, "moe_expert_capacity",
                       f"invalid arguments T={T} k={k} E={E} n_groups={n_groups} factor={factor}")
    return c


def moe_capacity(dims, n_groups, capacity, topk_idx, kept_idx, group_dropped, workspace,
                 stream=None):
    st = lib().moe_capacity(ctypes.byref(dims), int(n_groups), int(capacity),
                            _ptr(topk_idx, "topk_idx", torch.int32),
                            _ptr(kept_idx, "kept_idx", torch.int32),
                            _ptr(group_dropped, "group_dropped", torch.int32),
                            _ptr(workspace, "workspace"),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_capacity")


def moe_router_zloss(dims, logits, n_groups, group_z, workspace, stream=None):
    st = lib().moe_router_zloss(ctypes.byref(dims), _ptr(logits, "logits", torch.float32),
                                int(n_groups), _ptr(group_z, "group_z", torch.float32),
                                _ptr(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_router_zloss")


def moe_route_bwd_dense(dims, x, w_router, logits, topk_idx, topk_gate, dgate, pos, dx_perm,
                        n_groups, group_count, aux_coef, z_coef, dx, dw_router, dlogits,
                        workspace, stream=None):
    act = act_dtype(dims)
    st = lib().moe_route_bwd_dense(
        ctypes.byref(dims), _ptr(x, "x", act), _ptr(w_router, "w_router", torch.float32),
        _ptr(logits, "logits", torch.float32), _ptr(topk_idx, "topk_idx", torch.int32),
        _ptr(topk_gate, "topk_gate", torch.float32), _ptr(dgate, "dgate", torch.float32),
        _ptr(pos, "pos", torch.int32), _ptr(dx_perm, "dx_perm", act), int(n_groups),
        _ptr(group_count, "group_count", torch.int32), float(aux_coef), float(z_coef),
        _ptr(dx, "dx", act), _ptr(dw_router, "dw_router", torch.float32),
        _ptr(dlogits, "dlogits", torch.float32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_route_bwd_dense")


# ---------------------------------------------------------------- token-shuffle planning
def moe_coselect_cross(T, k, E, topk_idx_cur, topk_idx_next, coselect, stream=None):
    st = lib().moe_coselect_cross(int(T), int(k), int(E),
                                  _ptr(topk_idx_cur, "topk_idx_cur", torch.int32),
                                  _ptr(topk_idx_next, "topk_idx_next", torch.int32),
                                  _ptr(coselect, "coselect", torch.int32), _stream(stream))
    _check(st, "moe_coselect_cross")


def moe_shuffle_plan(T, k, E, G, topk_idx_cur, predictor, placement_next, topk_idx_next, owner,
                     group_tokens, stats, workspace, stream=None):
    pl = (ctypes.c_int32 * E)(*[int(v) for v in placement_next])
    st = lib().moe_shuffle_plan(int(T), int(k), int(E), int(G),
                                _ptr(topk_idx_cur, "topk_idx_cur", torch.int32),
                                _ptr(predictor, "predictor", torch.int32),
                                ctypes.cast(pl, ctypes.c_void_p),
                                _ptr(topk_idx_next, "topk_idx_next", torch.int32),
                                _ptr(owner, "owner", torch.int32),
                                _ptr(group_tokens, "group_tokens", torch.int32),
                                _ptr(stats, "stats", torch.int32), _ptr(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_shuffle_plan")


def moe_route_flips(T, k, E, topk_idx_a, topk_idx_b, flips, n_flips, stream=None):
    st = lib().moe_route_flips(int(T), int(k), int(E), _ptr(topk_idx_a, "topk_idx_a", torch.int32),
                               _ptr(topk_idx_b, "topk_idx_b", torch.int32),
                               _ptr(flips, "flips", torch.int32),
                               _ptr(n_flips, "n_flips", torch.int32), _stream(stream))
    _check(st, "moe_route_flips")
