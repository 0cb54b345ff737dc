"""One MoE layer's forward and backward as a sequence of C-ABI calls.

Buffers for every intermediate are allocated once (torch device memory) and
reused by each call, so a step enqueues kernels only.  The sequence is:

  forward:  moe_route -> moe_permute -> moe_grouped_swiglu_fwd -> moe_combine
  backward: moe_combine_bwd -> moe_grouped_swiglu_bwd -> moe_route_bwd

(moe_route_bwd also unpermutes and sums the expert input gradients).  With
gather=True the permutation is a plan only and the expert GEMMs read their
input rows from X through src_token (moe_grouped_swiglu_fwd_gather /
bwd_gather), so x_perm is never materialised; the results are identical.

Definitional variants: capacity_factor enables per-block expert capacity
(moe_capacity between the router and the permutation: dropped assignments get
no row), and aux_coef / z_coef add the balancing and z-loss gradients.  Either
switches the router backward to moe_route_bwd_dense; z_coef also computes the
per-block z-loss values (moe_router_zloss) in the forward.

fold_gate=True (bf16, gathered input, dims that moe_gate_folded_supported
accepts) moves the combine's gate onto the expert rows: the forward stores
h = g silu(a) b (moe_permute_gates, moe_expert_up_folded, moe_expert_down,
moe_combine without gates) and the backward reads dY through src_token
(moe_expert_dgrad_down_folded, moe_expert_dgrad_up, moe_expert_wgrad_folded,
moe_route_bwd_folded, which also sums the dgate parts; with the dense router
backward, or more than two parts per row, moe_dgate_from_parts sums them
first), so neither moe_combine_bwd nor dy_perm exists.
The results equal the unfolded layer's up to rounding.

Backward options of the expert call: wgrad_dtype=torch.float32 on a bf16 layer
keeps dW1, dW3, dW2 as the fp32 sums (not rounded to bf16), and
recompute=True hands the backward no saved a, b, h, so that it recomputes
them with the forward kernel (the forward still stores them here; the results
are the same bits).  Neither combines with fold_gate.
"""
from __future__ import annotations

import torch

from . import _lib as L


class MoELayer:
    def __init__(self, T: int, d: int, E: int, f: int, k: int, act: torch.dtype,
                 n_groups: int = 1, near_tie_eps: float = 1e-3, device="cuda",
                 gather: bool = False, capacity_factor=None, aux_coef: float = 0.0,
                 z_coef: float = 0.0, fold_gate: bool = False, wgrad_dtype=None,
                 recompute: bool = False):
        self.dims = L.make_dims(T, d, E, f, k, act)
        self.wgrad_dtype = act if wgrad_dtype is None else wgrad_dtype
        self.recompute = bool(recompute)
        if fold_gate and (self.wgrad_dtype != act or self.recompute):
            raise ValueError("fold_gate takes neither another wgrad_dtype nor recompute")
        if fold_gate and not (gather and L.moe_gate_folded_supported(self.dims)):
            raise ValueError("fold_gate needs gather=True and dims that "
                             "moe_gate_folded_supported accepts (bf16, one-pass weight gradients)")
        self.fold_gate = fold_gate
        self.act = act
        self.gather = gather
        self.capacity = (None if capacity_factor is None else
                         L.moe_expert_capacity(T, k, E, n_groups, capacity_factor))
        self.aux_coef = float(aux_coef)
        self.z_coef = float(z_coef)
        self.dense_bwd = self.capacity is not None or self.aux_coef != 0.0 or self.z_coef != 0.0
        self.n_groups = n_groups
        self.eps = near_tie_eps
        R = T * k
        dev = torch.device(device)
        e32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        ea = dict(dtype=act, device=dev)

        def empty(*shape, **kw):
            # never a NULL pointer, even for an empty batch (T = 0)
            t = torch.empty(max(shape[0], 1), *shape[1:], **kw)
            return t[:shape[0]]

        self.logits = empty(T, E, **e32)
        self.topk_idx = empty(T, k, **i32)
        self.topk_gate = empty(T, k, **e32)
        self.margin = empty(T, **e32)
        self.near_tie_count = empty(1, **i32)
        self.group_count = empty(n_groups, E, **i32)
        self.group_mean_prob = empty(n_groups, E, **e32)
        self.group_aux = empty(n_groups, **e32)
        self.expert_counts = empty(E, **i32)
        self.expert_offsets = empty(E + 1, **i32)
        self.pos = empty(T, k, **i32)
        self.src_token = empty(R, **i32)
        self.x_perm = empty(0 if gather else R, d, **ea)
        self.a = empty(R, f, **ea)
        self.b = empty(R, f, **ea)
        self.h = empty(R, f, **ea)
        self.y_perm = empty(R, d, **ea)
        self.y = empty(T, d, **ea)
        self.dy_perm = empty(0 if fold_gate else R, d, **ea)
        self.gate_perm = empty(R, **e32) if fold_gate else None
        self.dgate_part = (empty(R, L.moe_dgate_parts(self.dims), **e32) if fold_gate
                           else None)
        self.da = empty(R, f, **ea) if fold_gate else None
        self.db = empty(R, f, **ea) if fold_gate else None
        self.dgate = empty(T, k, **e32)
        self.dx_perm = empty(R, d, **ea)
        ew = dict(dtype=self.wgrad_dtype, device=dev)
        self.dw1 = empty(E, f, d, **ew)
        self.dw3 = empty(E, f, d, **ew)
        self.dw2 = empty(E, d, f, **ew)
        self.dx = empty(T, d, **ea)
        self.dwr = empty(E, d, **e32)
        self.kept_idx = empty(T, k, **i32) if self.capacity is not None else None
        self.group_dropped = empty(n_groups, **i32) if self.capacity is not None else None
        self.group_z = empty(n_groups, **e32) if self.z_coef != 0.0 else None
        self.dlogits = empty(T, E, **e32) if self.dense_bwd else None
        self.workspace = L.alloc_workspace(self.dims, n_groups, dev)
        if self.recompute:
            need = L.moe_grouped_swiglu_bwd_workspace_bytes(self.dims, True)
            if need > self.workspace.numel():
                self.workspace = torch.empty(need, dtype=torch.uint8, device=dev)

    # ------------------------------------------------------------------ forward
    def route(self, x, wr):
        L.moe_route(self.dims, x, wr, self.logits, self.topk_idx, self.topk_gate, self.margin,
                    self.eps, self.near_tie_count, self.n_groups, self.group_count,
                    self.group_mean_prob, self.group_aux, self.workspace)

    def forward_experts(self, x, w1, w3, w2):
        table = self.topk_idx
        if self.capacity is not None:
            L.moe_capacity(self.dims, self.n_groups, self.capacity, self.topk_idx, self.kept_idx,
                           self.group_dropped, self.workspace)
            table = self.kept_idx
        if self.z_coef != 0.0:
            L.moe_router_zloss(self.dims, self.logits, self.n_groups, self.group_z,
                               self.workspace)
        if self.fold_gate:
            L.moe_permute_gates(self.dims, table, self.topk_gate, self.expert_counts,
                                self.expert_offsets, self.pos, self.src_token, self.gate_perm,
                                self.workspace)
            L.moe_expert_up_folded(self.dims, x, self.src_token, self.expert_offsets,
                                   self.gate_perm, w1, w3, self.a, self.b, self.h)
            L.moe_expert_down(self.dims, self.h, self.expert_offsets, w2, self.y_perm)
            L.moe_combine(self.dims, self.y_perm, self.pos, None, self.y)
            return
        if self.gather:
            L.moe_permute(self.dims, table, self.expert_counts, self.expert_offsets,
                          self.pos, self.src_token, None, None, self.workspace)
            L.moe_grouped_swiglu_fwd_gather(self.dims, x, self.src_token, self.expert_offsets,
                                            w1, w3, w2, self.a, self.b, self.h, self.y_perm)
        else:
            L.moe_permute(self.dims, table, self.expert_counts, self.expert_offsets,
                          self.pos, self.src_token, x, self.x_perm, self.workspace)
            L.moe_grouped_swiglu_fwd(self.dims, self.x_perm, self.expert_offsets, w1, w3, w2,
                                     self.a, self.b, self.h, self.y_perm)
        L.moe_combine(self.dims, self.y_perm, self.pos, self.topk_gate, self.y)

    def forward(self, x, wr, w1, w3, w2, routing=None):
        """routing: optional (topk_idx, topk_gate) device tensors that replace the
        router's decision after it has run (used to compare the downstream
        steps on a routing fixed from outside)."""
        self.route(x, wr)
        if routing is not None:
            self.topk_idx.copy_(routing[0])
            self.topk_gate.copy_(routing[1])
        self.forward_experts(x, w1, w3, w2)
        return self.y

    # ------------------------------------------------------------------ backward
    def backward(self, dy, x, wr, w1, w3, w2):
        if self.fold_gate:
            L.moe_expert_dgrad_down_folded(self.dims, dy, self.src_token, self.expert_offsets,
                                           self.gate_perm, w2, self.a, self.b, self.da, self.db,
                                           self.dgate_part)
            # with more than two parts per row the router backward's dX threads
            # would each reload them all: sum them once instead
            parts_first = self.dense_bwd or L.moe_dgate_parts(self.dims) > 2
            if parts_first:
                L.moe_dgate_from_parts(self.dims, self.dgate_part, self.pos, self.dgate)
            L.moe_expert_dgrad_up(self.dims, self.da, self.db, self.expert_offsets, w1, w3,
                                  self.dx_perm)
            L.moe_expert_wgrad_folded(self.dims, x, dy, self.src_token, self.expert_offsets,
                                      self.h, self.da, self.db, self.dw1, self.dw3, self.dw2)
            if not parts_first:   # the router backward sums the parts into dgate itself
                L.moe_route_bwd_folded(self.dims, x, wr, self.topk_idx, self.topk_gate,
                                       self.dgate_part, self.expert_offsets, self.pos,
                                       self.src_token, self.dx_perm, self.dgate, self.dx,
                                       self.dwr, self.workspace)
                return self.dx
        else:
            self._experts_bwd(dy, x, w1, w3, w2)
        self._router_bwd(x, wr)
        return self.dx

    def _experts_bwd(self, dy, x, w1, w3, w2):
        L.moe_combine_bwd(self.dims, dy, self.y_perm, self.pos, self.topk_gate, self.dy_perm,
                          self.dgate)
        saved = (None, None, None) if self.recompute else (self.a, self.b, self.h)
        if self.gather:
            L.moe_grouped_swiglu_bwd_gather(self.dims, x, self.src_token, self.expert_offsets,
                                            w1, w3, w2, *saved, self.dy_perm, self.dx_perm,
                                            self.dw1, self.dw3, self.dw2, self.workspace,
                                            wgrad_dtype=self.wgrad_dtype)
        else:
            L.moe_grouped_swiglu_bwd(self.dims, self.x_perm, self.expert_offsets, w1, w3, w2,
                                     *saved, self.dy_perm, self.dx_perm, self.dw1, self.dw3,
                                     self.dw2, self.workspace, wgrad_dtype=self.wgrad_dtype)

    def _router_bwd(self, x, wr):
        if self.dense_bwd:
            L.moe_route_bwd_dense(self.dims, x, wr, self.logits, self.topk_idx, self.topk_gate,
                                  self.dgate, self.pos, self.dx_perm, self.n_groups,
                                  self.group_count, self.aux_coef, self.z_coef, self.dx,
                                  self.dwr, self.dlogits, self.workspace)
        else:
            L.moe_route_bwd(self.dims, x, wr, self.topk_idx, self.topk_gate, self.dgate,
                            self.expert_offsets, self.pos, self.src_token, self.dx_perm, self.dx,
                            self.dwr, self.workspace)
        return self.dx

    def step(self, x, wr, w1, w3, w2, dy):
        self.forward(x, wr, w1, w3, w2)
        self.backward(dy, x, wr, w1, w3, w2)
