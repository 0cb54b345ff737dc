"""Shared parity checks of the GPU layer against the CPU oracle.

check_route holds moe_route to the routing rules; exact_reference runs the
exact (fp64, unrounded, unfolded) oracle layer on a given routing together
with its first-order error bounds; layer_floats collects a MoELayer's float
outputs next to the matching exact values and bounds, so that check_floats
can hold every element to them.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O

from _util import TOL_ROUTER, dev, host, rel_err

EPS = 1e-3


def check_route(layer, x, wr, k, G=1, eps=EPS):
    """Run moe_route and hold it to the routing rules:
      * logits within 1e-4 (row-normwise) of the fp64 oracle;
      * expert sets identical wherever the oracle's margin is >= eps, and at a
        near-tie a set that is still a top-k of the oracle's logits to within
        fp32 resolution; slots in non-increasing logit order;
      * gates (compared per expert id on tokens with the same set), margins,
        the near-tie count and the per-block LB statistics.
    Returns (oracle route, mask of tokens routed to the same set)."""
    E = wr.shape[0]
    o = O.route(x, wr, k, eps)
    act = layer.act
    layer.route(dev(x, act), dev(wr, torch.float32))
    torch.cuda.synchronize()
    lg, idx = host(layer.logits), host(layer.topk_idx)
    gate, margin = host(layer.topk_gate), host(layer.margin)
    T = x.shape[0]
    if T == 0:
        assert int(host(layer.near_tie_count)[0]) == 0
        return o, np.zeros(0, bool)
    assert rel_err(lg, o["logits"]) <= TOL_ROUTER
    scale = float(np.sqrt(np.mean(o["logits"] ** 2))) or 1.0
    tol = 1e-5 * scale
    assert idx.min() >= 0 and idx.max() < E
    assert np.all(np.sort(idx, 1)[:, 1:] != np.sort(idx, 1)[:, :-1])  # no repeats
    same = np.all(np.sort(idx, 1) == np.sort(o["topk_idx"], 1), axis=1)
    clear = o["margin"] >= eps
    assert same[clear].all(), f"{(~same[clear]).sum()} clear-margin tokens routed differently"
    lo = o["logits"]
    for t in np.where(~same)[0]:
        chosen = idx[t]
        others = np.setdiff1d(np.arange(E), chosen)
        assert lo[t, chosen].min() >= lo[t, others].max() - tol, t
    ordered = np.take_along_axis(lo, idx.astype(np.int64), 1)
    assert np.all(np.diff(ordered, axis=1) <= tol)
    gd = np.zeros((T, E))
    go = np.zeros((T, E))
    np.put_along_axis(gd, idx.astype(np.int64), gate, 1)
    np.put_along_axis(go, o["topk_idx"].astype(np.int64), o["gates"], 1)
    assert rel_err(gd[same], go[same]) <= TOL_ROUTER
    if k < E:
        assert np.abs(margin[same] - o["margin"][same]).max() <= tol
    else:
        assert np.all(np.isinf(margin))
    ambiguous = int((np.abs(o["margin"] - eps) < tol).sum())
    assert abs(int(host(layer.near_tie_count)[0]) - o["near_tie_count"]) <= ambiguous
    s = O.lb_stats(lo, o["topk_idx"], E, G)
    n = T // G
    mism = [(~same[r * n:(r + 1) * n]).sum() for r in range(G)]
    cnt = host(layer.group_count)
    for r in range(G):
        assert np.abs(cnt[r] - s["count"][r]).sum() <= 2 * mism[r]
    assert rel_err(host(layer.group_mean_prob), s["P"]) <= TOL_ROUTER
    if sum(mism) == 0:
        assert np.array_equal(cnt, s["count"])
        assert rel_err(host(layer.group_aux), s["aux"]) <= TOL_ROUTER
    return o, same


def oracle_routing(o):
    return (dev(o["topk_idx"], torch.int32), dev(o["gates"].astype(np.float32), torch.float32))


def exact_reference(inp, k, routing, backward=True, act="bf16", capacity=None, lb_groups=1,
                    aux_coef=0.0, z_coef=0.0):
    """The exact oracle layer on `routing` (topk_idx, gates) and its bounds
    for storage unit roundoff 2**-8 (bf16) or 2**-24 (fp32)."""
    o_f = O.layer_forward(inp["x"], inp["wr"], inp["w1"], inp["w3"], inp["w2"], k,
                          routing=routing, capacity=capacity, lb_groups=lb_groups)
    o_b = None
    if backward:
        o_b = O.layer_backward(inp["x"], inp["wr"], inp["w1"], inp["w3"], inp["w2"], o_f,
                               inp["dy"], aux_coef, z_coef)
    u = O.U_BF16 if act == "bf16" else O.U_F32
    B = O.layer_error_bounds(inp["x"], inp["wr"], inp["w1"], inp["w3"], inp["w2"], o_f, o_b,
                             inp.get("dy"), u=u, aux_coef=aux_coef, z_coef=z_coef)
    return o_f, o_b, B


def check_plan(layer, o_f):
    """Counts, offsets, positions and source tokens bit-exact."""
    R = int(o_f["offsets"][-1])
    assert np.array_equal(host(layer.expert_counts), o_f["counts"])
    assert np.array_equal(host(layer.expert_offsets), o_f["offsets"])
    assert np.array_equal(host(layer.pos), o_f["pos"])
    assert np.array_equal(host(layer.src_token)[:R], o_f["src"][:R])


def layer_floats(layer, o_f, o_b, B):
    """(got, exact, bounds) dicts over every float output the layer holds.
    With the gate folded onto the expert rows, h holds g h and y_perm holds
    g y_perm: both are held to the exact values times the row gate, with the
    bounds scaled the same way (the gate is an exact fp32 value)."""
    R = int(o_f["offsets"][-1])
    got, ex, bd = {}, {}, {}
    g_row = None
    if layer.fold_gate:
        g_row = np.zeros(o_f["x_perm"].shape[0])
        live = o_f["pos"] >= 0
        g_row[o_f["pos"][live]] = o_f["gates"][live].astype(np.float32)
        gp = host(layer.gate_perm)[:R]
        assert np.array_equal(gp, g_row[:R].astype(np.float32))
    for key in ("a", "b", "h", "y_perm"):
        got[key] = host(getattr(layer, key))[:R]
        ex[key], bd[key] = o_f[key][:R], B[key][:R]
        if g_row is not None and key in ("h", "y_perm"):
            ex[key] = ex[key] * g_row[:R, None]
            bd[key] = bd[key] * g_row[:R, None]
    got["y"], ex["y"], bd["y"] = host(layer.y), o_f["y"], B["y"]
    if o_b is None:
        return got, ex, bd
    rows = ["dx_perm"]
    if not layer.fold_gate and layer.dy_perm.shape[0]:
        rows.append("dy_perm")
    if layer.da is not None:
        rows += ["da", "db"]
    for key in rows:
        got[key] = host(getattr(layer, key))[:R]
        ex[key], bd[key] = o_b[key][:R], B[key][:R]
    for key in ("dgate", "dx", "dw1", "dw3", "dw2", "dwr"):
        got[key], ex[key], bd[key] = host(getattr(layer, key)), o_b[key], B[key]
    if getattr(layer, "dlogits", None) is not None:
        got["dlogits"], ex["dlogits"], bd["dlogits"] = (host(layer.dlogits), o_b["dlogits"],
                                                        B["dlogits"])
    return got, ex, bd


def bound_only_keys(cfg):
    """Outputs held to the bound alone:
      * the logit gradient dl[t, S_j] = g_j (dg_j - sum_i g_i dg_i), whose
        difference cancels wherever a token's dgate values are close, so that
        the bf16 rounding of the expert path upstream of dgate reaches 3-5e-2
        of it (row-normwise) in any bf16-storage computation;
      * the expert weight gradients of the workloads with clustered hidden
        states, whose sums over many nearly parallel rows cancel (2-4e-2 by
        rounding alone there)."""
    return ("dlogits",) + (("dw1", "dw3", "dw2") if cfg.x_kind == "mixture" else ())


def cancellation(o_f, o_b, keys):
    """How much the exact sums of the bound-only outputs cancel: per row,
    max_j sum|terms| / max(max_j |sum|, rms of the tensor), summarised as the
    median and the largest over rows (the row-normwise error that a
    relative perturbation u of every term can cause is u times this).
    Returns {key: (median, max)} for the keys among dw1, dw3, dw2, dlogits."""
    out = {}
    off = o_f["offsets"]
    E = len(off) - 1
    pairs = {"dw1": ("da", o_f["x_perm"]), "dw3": ("db", o_f["x_perm"]),
             "dw2": ("dy_perm", o_f["h"])}
    for key in keys:
        if key in pairs:
            op, right = pairs[key]
            ratios = []
            ref = np.abs(o_b[key])
            rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
            for e in range(E):
                s = slice(int(off[e]), int(off[e + 1]))
                if off[e + 1] == off[e]:
                    continue
                terms = np.abs(o_b[op][s]).T @ np.abs(right[s])
                ratios.append(terms.max(axis=1) / np.maximum(ref[e].max(axis=1), rms))
            r = np.concatenate(ratios) if ratios else np.zeros(1)
        elif key == "dlogits":
            # dl[t, S_j] = g_j (dg_j - sum_i g_i dg_i)
            g, dg = o_f["gates"], o_b["dgate"]
            inner = (g * np.abs(dg)).sum(axis=1, keepdims=True)
            terms = (g * (np.abs(dg) + inner)).max(axis=1)
            ref = np.abs(o_b["dlogits"])
            rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
            r = terms / np.maximum(ref.max(axis=1), rms)
        else:
            continue
        out[key] = (float(np.median(r)), float(r.max()))
    return out

