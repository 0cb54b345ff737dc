"""Benchmark: MoE layer forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

One step is one full pass of the layer's hot path over one batch of synthetic
tokens: moe_route -> moe_permute -> moe_expert_up -> moe_expert_down ->
moe_combine -> moe_combine_bwd -> moe_expert_dgrad_down -> moe_expert_dgrad_up
-> moe_expert_wgrad -> moe_route_bwd (the kernel-level phases of
moe_grouped_swiglu_fwd/bwd, so each GEMM kernel can be timed on its own).
By default the permutation is a plan only and moe_expert_up / moe_expert_wgrad
read their input rows from X through src_token (the *_gather calls, reported
as moe_permute_plan, moe_expert_up_gather, moe_expert_wgrad_gather);
--no-gather materialises x_perm instead.  Both compute the same bits.
Where the dims allow it (bf16 with one-pass weight gradients: C2-C5) the
gate is folded onto the expert rows by default: moe_permute_gates ->
moe_expert_up_folded -> moe_expert_down -> moe_combine (no gates) ->
moe_expert_dgrad_down_folded -> moe_expert_dgrad_up -> moe_expert_wgrad_folded
-> moe_route_bwd_folded (which sums the dgate parts; with more than two parts
per row moe_dgate_from_parts -> moe_route_bwd instead), with no
moe_combine_bwd and no dy_perm; --no-fold keeps the gate in the combine.
config.gate says which.
Inputs and weights are resident in HBM before timing starts.  Prints one JSON
line.

Per-call durations are taken live with HIP events on the stream the library
launches on; the dominant call's algorithmic bytes (or flops) per launch over
its mean duration give the roofline fraction.  The CPU baseline is the fp64
oracle, timed on the host cores on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/s on 1 MI355X; grouped-GEMM % of bf16 MFMA peak"
PEAK_HBM = 8.0e12          # bytes/s
PEAK_MFMA = {"bf16": 2.5e15, "f32": 157.3e12}   # dense matrix peaks (fp32: vector/matrix fp32)


def algorithmic_work(cfg, R=None, fold=False, parts=1):
    """Per-call algorithmic (flops, bytes, kernels): what each call must compute
    and move by its C-ABI contract (inputs read once, outputs written once).
    R: expert rows (T k, or fewer when a capacity drops assignments).  fold:
    the gate sits on the expert rows (the combine reads no gates); parts: the
    dgate parts per row of the folded backward."""
    T, d, E, f, k = cfg.T, cfg.d, cfg.E, cfg.f, cfg.k
    R = T * k if R is None else R
    s = 2 if cfg.act == "bf16" else 4
    i4 = 4
    Wf = E * d * f * s          # one of W1, W3, W2
    gates = 0 if fold else T * k * 4
    return {
        # gate folded onto the expert rows: dY read through src_token, no dy_perm
        "moe_permute_gates": (0, T * k * (i4 + 4) + 2 * R * i4 + R * 4 + (2 * E + 1) * i4, 2),
        "moe_expert_up_folded": (4 * R * d * f,
                                 R * d * s + R * (i4 + 4) + 2 * Wf + 3 * R * f * s, 1),
        "moe_expert_dgrad_down_folded": (2 * R * d * f + 2 * R * f,
                                         R * d * s + R * (i4 + 4) + Wf + 4 * R * f * s
                                         + R * parts * 4, 1),
        "moe_dgate_from_parts": (R * parts, R * parts * 4 + T * k * (i4 + 4), 1),
        "moe_route_bwd_folded": (4 * R * d + R * parts,
                                 T * d * s + E * d * 4 + R * d * s + T * d * s + E * d * 4
                                 + T * k * 16 + R * parts * 4 + R * 8, 4),
        "moe_expert_wgrad_folded": (6 * R * d * f,
                                    2 * R * d * s + R * i4 + 3 * R * f * s + 3 * Wf, 1),
        "moe_route": (2 * T * d * E,
                      T * d * s + E * d * 4 + T * E * 4 + T * k * (i4 + 4) + T * 4, 2),
        "moe_permute": (0, T * k * i4 + T * d * s + R * d * s + 2 * R * i4 + (2 * E + 1) * i4, 4),
        # plan only (gathered expert input): indices in, counts/offsets/pos/src out
        "moe_permute_plan": (0, T * k * i4 + 2 * R * i4 + (2 * E + 1) * i4, 2),
        "moe_expert_up": (4 * R * d * f, R * d * s + 2 * Wf + 3 * R * f * s, 1),
        "moe_expert_up_gather": (4 * R * d * f, R * d * s + R * i4 + 2 * Wf + 3 * R * f * s, 1),
        "moe_expert_down": (2 * R * d * f, R * f * s + Wf + R * d * s, 1),
        "moe_combine": (2 * R * d, R * d * s + T * d * s + T * k * i4 + gates, 1),
        "moe_combine_bwd": (2 * R * d, T * d * s + 2 * R * d * s + T * k * (i4 + 8), 1),
        "moe_expert_dgrad_down": (2 * R * d * f, R * d * s + Wf + 4 * R * f * s, 1),
        "moe_expert_dgrad_up": (4 * R * d * f, 2 * R * f * s + 2 * Wf + R * d * s, 1),
        "moe_expert_wgrad": (6 * R * d * f, 2 * R * d * s + 3 * R * f * s + 3 * Wf, None),
        "moe_expert_wgrad_gather": (6 * R * d * f, 2 * R * d * s + R * i4 + 3 * R * f * s + 3 * Wf,
                                    None),
        "moe_route_bwd": (4 * R * d, T * d * s + E * d * 4 + R * d * s + T * d * s + E * d * 4
                          + T * k * 12 + R * 8, 4),
        # definitional variants
        "moe_capacity": (0, 2 * T * k * i4, 1),
        "moe_router_zloss": (3 * T * E, T * E * 4, 1),
        "moe_route_bwd_dense": (4 * T * E * d, T * d * s + E * d * 4 + T * E * 8 + T * k * 16
                                + R * d * s + T * d * s + E * d * 4, 4),
    }


GEMM_CALLS = ("moe_expert_up", "moe_expert_down", "moe_expert_dgrad_down",
              "moe_expert_dgrad_up", "moe_expert_wgrad", "moe_expert_up_gather",
              "moe_expert_wgrad_gather", "moe_expert_up_folded", "moe_expert_dgrad_down_folded",
              "moe_expert_wgrad_folded")
WGRAD_CALLS = ("moe_expert_wgrad", "moe_expert_wgrad_gather")


def wgrad_kernels(dm):
    """Kernels moe_expert_wgrad enqueues for these dims, as the library reports
    (1, or 2 when it splits the expert rows and adds a reduction)."""
    import ctypes
    import top_routing_grouped_router_amd._lib as L
    return int(L.lib().moe_expert_wgrad_launches(ctypes.byref(dm)))


def roofline_entry(flops, nbytes, seconds, act):
    peak_f = PEAK_MFMA[act]
    if flops / peak_f > nbytes / PEAK_HBM:
        achieved = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_f / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / (peak_f / 1e12), 4)}
    achieved = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
            "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "moe_expert_up": "gemm_bf16.hip", "moe_expert_down": "gemm_bf16.hip",
    "moe_expert_up_gather": "gemm_bf16.hip", "moe_expert_wgrad_gather": "gemm_bf16.hip",
    "moe_permute_plan": "permute.hip",
    "moe_expert_dgrad_down": "gemm_bf16.hip", "moe_expert_dgrad_up": "gemm_bf16.hip",
    "moe_expert_wgrad": "gemm_bf16.hip", "moe_route": "route.hip", "moe_permute": "permute.hip",
    "moe_combine": "combine.hip", "moe_combine_bwd": "combine.hip",
    "moe_route_bwd": "route_bwd.hip", "moe_permute_gates": "permute.hip",
    "moe_expert_up_folded": "gemm_bf16.hip", "moe_expert_dgrad_down_folded": "gemm_bf16.hip",
    "moe_expert_wgrad_folded": "gemm_bf16.hip", "moe_dgate_from_parts": "combine.hip",
    "moe_route_bwd_folded": "route_bwd.hip",
}


def source_digest(name):
    import hashlib
    path = os.path.join(ROOT, "top_routing_grouped_router_amd", "csrc", name)
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(workload, call):
    """HBM bytes per launch of `call` at `workload` from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading
    for a plain copy of known size), or None when there is none or the
    kernel's source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload, {}).get(call)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest(KERNEL_SOURCES[call]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, inp, budget_s=20.0):
    """The oracle as it stands (fp64 numpy), timed on the host cores on the same
    workload.  Whole steps of the full batch when one step takes under ~budget/2
    seconds; otherwise the first `n` tokens of the batch (same weights), n sized
    from a short probe.  Repeats until budget_s is spent (at least once)."""
    import threadpoolctl
    from oracle import moe_oracle as O
    cores = len(os.sched_getaffinity(0))
    threadpoolctl.threadpool_limits(cores)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    def step(n):
        sl = slice(0, n)
        fwd = O.layer_forward(inp["x"][sl], inp["wr"], inp["w1"], inp["w3"], inp["w2"], cfg.k)
        if cfg.backward:
            O.layer_backward(inp["x"][sl], inp["wr"], inp["w1"], inp["w3"], inp["w2"], fwd,
                             inp["dy"][sl])

    n = cfg.T
    probe = min(cfg.T, 512)
    t0 = time.perf_counter()
    step(probe)
    per_token = (time.perf_counter() - t0) / probe
    if per_token * cfg.T > budget_s / 2:
        n = max(probe, int(budget_s / 3 / per_token) // 256 * 256)
        n = min(n, cfg.T)
    t0 = time.perf_counter()
    steps = 0
    while True:
        step(n)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (steps + 1) / steps > 1.5 * budget_s:
            break
    what = "full batch" if n == cfg.T else f"first {n} of {cfg.T} tokens"
    return {"value": round(n * steps / el, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": model, "affinity_cores": cores,
            "sample": f"{steps} step(s) of {cfg.name} over the {what} (fwd"
                      f"{'+bwd' if cfg.backward else ''}), fp64 numpy, {el:.1f} s"}


def workload_reports(steps):
    """The index products the workloads are defined by, computed by the
    library on each workload's own seeded inputs (the router's routing, not
    the oracle's):
      * C3: the near-tie share at margin 1e-3 ([LAYOUT] Finding 3) and the
        share of normalised margins (gap / spread of the token's logits) under
        0.01 (Finding 4's measure);
      * C2: per-block balancing statistics for G = 1, 2, 4, 8 blocks
        ([LAYOUT] Two Kinds of Layout Effects; [REVISIT] Sec. 2.2 outer
        batches): aux per block and the largest and smallest E f and E P;
      * C4 and C5: the deduplicated dispatch plan for each of the workload's
        group counts under contiguous and correlated (greedy co-selection,
        fit on another batch) placement ([COUPLING] Table I): share of tokens
        whose experts sit in one group, distinct destinations per token, and
        rows removed; plus C4's share of tokens whose top-2 pair is among the
        20 most frequent pairs (about 1% of the pairs)."""
    import torch
    from synth import get_config, make_layer_inputs
    import top_routing_grouped_router_amd._lib as L
    i32 = dict(dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    rep = {}

    def route(cfg, x_np, wr_np, G):
        act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
        dm = L.make_dims(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act)
        ws = L.alloc_workspace(dm, G)
        x = torch.from_numpy(x_np).to("cuda", act)
        wr = torch.from_numpy(wr_np).cuda()
        T, E, k = cfg.T, cfg.E, cfg.k
        o = {"logits": torch.empty(T, E, **f32), "idx": torch.empty(T, k, **i32),
             "gate": torch.empty(T, k, **f32), "margin": torch.empty(T, **f32),
             "ntc": torch.empty(1, **i32), "count": torch.empty(G, E, **i32),
             "P": torch.empty(G, E, **f32), "aux": torch.empty(G, **f32)}
        L.moe_route(dm, x, wr, o["logits"], o["idx"], o["gate"], o["margin"], 1e-3, o["ntc"], G,
                    o["count"], o["P"], o["aux"], ws)
        torch.cuda.synchronize()
        return o

    c3 = get_config("c3")
    inp = make_layer_inputs(c3, parts=("x", "wr"))
    r = route(c3, inp["x"], inp["wr"], 1)
    lg = r["logits"].cpu().numpy().astype(np.float64)
    mg = r["margin"].cpu().numpy().astype(np.float64)
    spread = lg.max(1) - lg.min(1)
    norm = mg / np.where(spread > 0, spread, 1.0)
    rep["c3_near_ties"] = {"eps": 1e-3, "tokens": int(r["ntc"].item()), "of": c3.T,
                           "fraction": round(int(r["ntc"].item()) / c3.T, 4),
                           "normalised_margin_below_0.01": round(float((norm < 0.01).mean()), 4)}

    c2 = get_config("c2")
    inp = make_layer_inputs(c2, parts=("x", "wr"))
    lb = {}
    for G in c2.lb_groups:
        r = route(c2, inp["x"], inp["wr"], G)
        cnt = r["count"].cpu().numpy().astype(np.float64)
        fE = cnt / (c2.T // G * c2.k) * c2.E
        PE = r["P"].cpu().numpy().astype(np.float64) * c2.E
        lb[f"G{G}"] = {"aux": [round(float(v), 5) for v in r["aux"].cpu().numpy()],
                       "E_f_max": round(float(fE.max()), 4), "E_f_min": round(float(fE.min()), 4),
                       "E_P_max": round(float(PE.max()), 4), "E_P_min": round(float(PE.min()), 4)}
    rep["c2_lb_stats"] = lb

    dd = {}
    for name in ("c4", "c5"):
        cfg = get_config(name)
        inp = make_layer_inputs(cfg, parts=("x", "wr"))
        fit = make_layer_inputs(cfg, batch_seed=1, parts=("x",))
        idx = route(cfg, inp["x"], inp["wr"], 1)["idx"]
        idx_fit = route(cfg, fit["x"], inp["wr"], 1)["idx"]
        T, k, E = cfg.T, cfg.k, cfg.E
        W = torch.empty(E, E, **i32)
        L.moe_coselect(T, k, E, idx_fit, W)
        torch.cuda.synchronize()
        W_fit = W.cpu().numpy().astype(np.int64)
        if k == 2:
            pairs = np.sort(idx.cpu().numpy(), axis=1)
            _, cnts = np.unique(pairs[:, 0] * E + pairs[:, 1], return_counts=True)
            dd[f"{name}_top20_pair_token_share"] = round(float(np.sort(cnts)[::-1][:20].sum() / T),
                                                         4)
        for G in cfg.plan_groups:
            dm = L.make_dims(T, 64, E, 64, k, torch.bfloat16)
            ws = L.alloc_workspace(dm, G)
            for kind, pl in (("contiguous", [e * G // E for e in range(E)]),
                             ("correlated", L.moe_placement_greedy(E, G, W_fit))):
                out = {"n_dest": torch.empty(T, **i32), "group_rows": torch.empty(G, **i32),
                       "group_offsets": torch.empty(G + 1, **i32),
                       "row_token": torch.empty(T * k, **i32),
                       "assign_row": torch.empty(T, k, **i32), "stats": torch.empty(4, **i32)}
                L.moe_dispatch_plan(T, k, E, G, idx, pl, out["n_dest"], out["group_rows"],
                                    out["group_offsets"], out["row_token"], out["assign_row"],
                                    out["stats"], ws)
                torch.cuda.synchronize()
                rows, removed, single, _ = (int(v) for v in out["stats"].cpu().tolist())
                dd[f"{name}_G{G}_{kind}"] = {
                    "same_group_share": round(single / T, 4),
                    "destinations_per_token": round(rows / T, 4),
                    "rows_removed_share": round(removed / (T * k), 4)}
    rep["dedup_plans"] = dd
    return rep


def ep_dispatch(cfg, layer, x, wr, steps):
    """Expert-parallel dispatch emulated on one GPU for each placement group
    count of the workload, under contiguous placement and under the greedy
    correlated placement fitted on the co-selection of another batch: the
    dedup plan, the pack of one row per (group, token) and the receivers'
    expansion into x_perm, each timed with HIP events over `steps` launches.
    Bytes per pack: rows read + rows written (+ row ids); per expand: T k rows
    read + written (+ ids)."""
    import torch
    import top_routing_grouped_router_amd._lib as L
    T, k, E, d = cfg.T, cfg.k, cfg.E, cfg.d
    s = 2 if cfg.act == "bf16" else 4
    dm = layer.dims
    from synth import make_layer_inputs
    i32 = dict(dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    # route another batch with the same router to fit the correlated placement
    x_fit = torch.from_numpy(make_layer_inputs(cfg, batch_seed=1, parts=("x",))["x"]).to(
        "cuda", x.dtype)
    idx_fit = torch.empty(T, k, **i32)
    L.moe_route(dm, x_fit, wr, torch.empty(T, E, **f32), idx_fit, torch.empty(T, k, **f32),
                torch.empty(T, **f32), 1e-3, torch.empty(1, **i32), 1, torch.empty(1, E, **i32),
                torch.empty(1, E, **f32), torch.empty(1, **f32), layer.workspace)
    W = torch.empty(E, E, **i32)
    L.moe_coselect(T, k, E, idx_fit, W)
    torch.cuda.synchronize()
    W_fit = W.cpu().numpy().astype(np.int64)
    res = {}
    for G, kind in [(G, kind) for G in cfg.plan_groups for kind in ("contiguous", "correlated")]:
        pl = ([e * G // E for e in range(E)] if kind == "contiguous" else
              L.moe_placement_greedy(E, G, W_fit))
        out = {"n_dest": torch.empty(T, **i32), "group_rows": torch.empty(G, **i32),
               "group_offsets": torch.empty(G + 1, **i32), "row_token": torch.empty(T * k, **i32),
               "assign_row": torch.empty(T, k, **i32), "stats": torch.empty(4, **i32)}
        ws = torch.empty(L.workspace_bytes(dm, G), dtype=torch.uint8, device="cuda")
        send = torch.empty(T * k, d, dtype=x.dtype, device="cuda")
        xp = torch.empty(T * k, d, dtype=x.dtype, device="cuda")
        fns = {
            "plan": lambda: L.moe_dispatch_plan(T, k, E, G, layer.topk_idx, pl, out["n_dest"],
                                                out["group_rows"], out["group_offsets"],
                                                out["row_token"], out["assign_row"],
                                                out["stats"], ws),
            "pack": lambda: L.moe_dispatch_pack(dm, G, x, out["group_offsets"], out["row_token"],
                                                send),
            "expand": lambda: L.moe_dispatch_expand(dm, send, out["assign_row"], layer.pos, xp),
        }
        times = {}
        for name, fn in fns.items():
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            times[name] = a.elapsed_time(b) / steps * 1e-3
        rows = int(out["stats"][0].item())
        pack_b = rows * d * s * 2 + rows * 4
        exp_b = T * k * d * s * 2 + T * k * 8
        res[f"G{G}_{kind}"] = {
            "rows": rows, "rows_removed": T * k - rows,
            "plan_us": round(times["plan"] * 1e6, 1),
            "pack_us": round(times["pack"] * 1e6, 1),
            "pack_GBps": round(pack_b / times["pack"] / 1e9, 1),
            "expand_us": round(times["expand"] * 1e6, 1),
            "expand_GBps": round(exp_b / times["expand"] / 1e9, 1)}
    return res


def token_shuffle(cfg, layer, x, wr, steps):
    """Token-shuffle planning on one GPU for each placement group count of the
    workload: two layers' routes (the workload's router and a second router
    drawn from another seed, on the same hidden states), cross-layer counts fit
    on another batch of the workload, then the planner on this batch with the
    next layer's experts placed contiguously or by greedy co-selection (itself
    fit on the other batch).  Reports Table I's local next-layer assignments
    when tokens are moved to the predicted owner versus when they stay home,
    the spread of tokens per owner, and the planner's time (HIP events)."""
    import torch
    from synth import make_layer_inputs
    import top_routing_grouped_router_amd._lib as L
    T, k, E = cfg.T, cfg.k, cfg.E
    dm = layer.dims
    act = x.dtype
    i32 = dict(dtype=torch.int32, device="cuda")
    wr2 = torch.from_numpy(make_layer_inputs(cfg, seed=1, parts=("wr",))["wr"]).cuda()
    x_fit = torch.from_numpy(make_layer_inputs(cfg, batch_seed=1, parts=("x",))["x"]).to(
        "cuda", act)
    ws = torch.empty(L.workspace_bytes(dm, max(cfg.plan_groups)), dtype=torch.uint8,
                     device="cuda")

    def route(xx, w):
        lg = torch.empty(T, E, device="cuda")
        idx = torch.empty(T, k, **i32)
        gate = torch.empty(T, k, device="cuda")
        mg = torch.empty(T, device="cuda")
        ntc = torch.empty(1, **i32)
        L.moe_route(dm, xx, w, lg, idx, gate, mg, 1e-3, ntc, 1, None, None, None, ws)
        return idx

    fit_cur, fit_nxt = route(x_fit, wr), route(x_fit, wr2)
    cur, nxt = route(x, wr), route(x, wr2)
    W = torch.empty(E, E, **i32)
    L.moe_coselect_cross(T, k, E, fit_cur, fit_nxt, W)
    Wn = torch.empty(E, E, **i32)
    L.moe_coselect(T, k, E, fit_nxt, Wn)
    torch.cuda.synchronize()
    Wn_host = Wn.cpu().numpy().astype(np.int64)
    cond = W.cpu().numpy() / np.maximum(W.cpu().numpy().sum(1, keepdims=True) / k, 1)
    res = {"strong_pairs_pct": round(100.0 * float((cond > 0.3).mean()), 2)}
    for G in cfg.plan_groups:
        for name, pl in (("contiguous", [e * G // E for e in range(E)]),
                         ("correlated", L.moe_placement_greedy(E, G, Wn_host))):
            owner = torch.empty(T, **i32)
            gt = torch.empty(G, **i32)
            st = torch.empty(2, **i32)

            def plan():
                L.moe_shuffle_plan(T, k, E, G, cur, W, pl, nxt, owner, gt, st, ws)

            plan()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                plan()
            b.record()
            torch.cuda.synchronize()
            moved, stays = (int(v) for v in st.cpu().tolist())
            tokens = gt.cpu().numpy()
            res[f"G{G}_{name}"] = {
                "local_moved_pct": round(100.0 * moved / (T * k), 1),
                "local_stays_pct": round(100.0 * stays / (T * k), 1),
                "owner_tokens_max_over_mean": round(float(tokens.max()) / (T / G), 2),
                "plan_us": round(a.elapsed_time(b) / steps * 1e3, 1)}
    return res


def fragility(cfg, layer, x, wr, steps):
    """Routing-fragility probe: one router weight (a seeded expert, its
    largest-magnitude input weight) moved by m units in the last place of fp32,
    the router run again, and the tokens whose expert set changed
    (moe_route_flips) set against their margins in the unmoved run.  Reports,
    per m, the flip count, the largest logit shift |x[t,i] dw|, the share of
    flips whose margin is within that shift, the median normalised margin of
    flipped and kept tokens, and how much more often the 10% smallest margins
    flip than the rest."""
    import torch
    import top_routing_grouped_router_amd._lib as L
    T, k, E = cfg.T, cfg.k, cfg.E
    dm = layer.dims
    i32 = dict(dtype=torch.int32, device="cuda")
    ws = layer.workspace
    rng = np.random.default_rng(7)
    w_host = wr.cpu().numpy()
    e = int(rng.integers(0, E))
    i = int(np.argmax(np.abs(w_host[e])))

    def route(w):
        lg = torch.empty(T, E, device="cuda")
        idx = torch.empty(T, k, **i32)
        gate = torch.empty(T, k, device="cuda")
        mg = torch.empty(T, device="cuda")
        ntc = torch.empty(1, **i32)
        L.moe_route(dm, x, w, lg, idx, gate, mg, 1e-3, ntc, 1, None, None, None, ws)
        return idx, mg, lg

    base_idx, base_margin, base_lg = route(wr)
    lg = base_lg.cpu().numpy().astype(np.float64)
    spread = lg.max(1) - lg.min(1)
    margin = base_margin.cpu().numpy().astype(np.float64)
    norm = np.where(spread > 0, margin / np.where(spread > 0, spread, 1.0), np.inf)
    xcol = x[:, i].float().cpu().numpy().astype(np.float64)
    res = {"weight": [e, i]}
    flips = torch.empty(T, **i32)
    n = torch.empty(1, **i32)
    for m in (1, 1 << 10, 1 << 20):
        v = np.float32(w_host[e, i])
        bits = np.array([v], dtype=np.float32).view(np.int32)[0]
        # toward +inf: the magnitude grows for positive values, shrinks for negative
        bits = bits + m if v > 0 else bits - m
        wn = w_host.copy()
        wn[e, i] = np.array([bits], dtype=np.int32).view(np.float32)[0]
        idx_n, _, _ = route(torch.from_numpy(wn).cuda())
        L.moe_route_flips(T, k, E, base_idx, idx_n, flips, n)
        torch.cuda.synchronize()
        fl = flips.cpu().numpy().astype(bool)
        shift = np.abs(xcol * (float(wn[e, i]) - float(v)))
        small = norm <= np.quantile(norm, 0.1)
        rate_small = fl[small].mean() if small.any() else 0.0
        rate_rest = fl[~small].mean() if (~small).any() else 0.0
        res[str(m)] = {
            "flips": int(fl.sum()), "max_logit_shift": float(f"{shift.max():.3e}"),
            "flips_within_shift_pct": (round(100.0 * float((margin[fl] <= shift[fl] + 1e-5).mean()),
                                             1) if fl.any() else None),
            "median_norm_margin_flipped": (float(f"{np.median(norm[fl]):.3e}") if fl.any()
                                           else None),
            "median_norm_margin_kept": float(f"{np.median(norm[~fl]):.3e}"),
            "smallest_decile_flip_rate_ratio": (round(float(rate_small / rate_rest), 1)
                                                if rate_rest > 0 else None)}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        L.moe_route_flips(T, k, E, base_idx, idx_n, flips, n)
    b.record()
    torch.cuda.synchronize()
    res["route_flips_us"] = round(a.elapsed_time(b) / steps * 1e3, 1)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5"],
                    help="c5 (the largest single-GPU workload) by default; the others are "
                         "parity cases that can be timed too")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="bytes written before every timed step to evict L2 and MALL "
                         "(outside the step's events); 0 disables the flushed headline")
    ap.add_argument("--no-reports", action="store_true",
                    help="skip the per-workload reports (C3 near-ties, C2 balancing "
                         "statistics per group count, C4/C5 dedup plans)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-gather", action="store_true",
                    help="materialise x_perm in moe_permute and run the expert GEMMs on it "
                         "instead of gathering the expert input rows from X")
    ap.add_argument("--ep", action="store_true",
                    help="also time the expert-parallel dispatch emulation (dedup plan, pack, "
                         "expand) for the workload's placement group counts; adds an "
                         "'ep_dispatch' object to the JSON line")
    ap.add_argument("--no-fold", action="store_true",
                    help="keep the gate in the combine (moe_combine_bwd and dy_perm) even "
                         "where the folded path is supported")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph (per-call times "
                         "still come from eager launches)")
    ap.add_argument("--fragility", action="store_true",
                    help="also run the routing-fragility probe (one router weight moved by "
                         "1, 2^10 and 2^20 ulps; flips against margins); adds a 'fragility' "
                         "object")
    ap.add_argument("--shuffle", action="store_true",
                    help="also run the token-shuffle planner (cross-layer counts of two routers, "
                         "owner prediction, local next-layer assignments) for the workload's "
                         "placement group counts; adds a 'token_shuffle' object")
    ap.add_argument("--capacity-factor", type=float, default=None,
                    help="definitional variant: per-block expert capacity with dropping "
                         "(moe_capacity before the permutation, moe_route_bwd_dense after)")
    ap.add_argument("--aux-coef", type=float, default=0.0,
                    help="definitional variant: GShard balancing-loss gradient coefficient")
    ap.add_argument("--z-coef", type=float, default=0.0,
                    help="definitional variant: router z-loss coefficient (values and gradient)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a "
                         "known-size kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of tokens; --gpus {args.gpus} is not "
              "supported (the MoE layer path here runs on a single GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import get_config, make_layer_inputs
    from top_routing_grouped_router_amd import MoELayer
    import top_routing_grouped_router_amd._lib as L

    cfg = get_config(args.workload)
    inp = make_layer_inputs(cfg, with_dy=True)
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a, dt):
        return torch.from_numpy(a).to(dev, dt).contiguous()

    x, dy = up(inp["x"], act), up(inp["dy"], act)
    wr = up(inp["wr"], torch.float32)
    w1, w3, w2 = up(inp["w1"], act), up(inp["w3"], act), up(inp["w2"], act)
    G = max(cfg.lb_groups)
    gather = not args.no_gather
    fold = (gather and not args.no_fold and
            L.moe_gate_folded_supported(L.make_dims(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act)))
    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=G, gather=gather,
                     capacity_factor=args.capacity_factor, aux_coef=args.aux_coef,
                     z_coef=args.z_coef, fold_gate=fold)
    dm = layer.dims
    table = layer.kept_idx if layer.capacity is not None else layer.topk_idx

    da = torch.empty_like(layer.a)
    db = torch.empty_like(layer.b)
    calls = [
        ("moe_route", lambda: layer.route(x, wr)),
        ("moe_capacity", lambda: L.moe_capacity(dm, G, layer.capacity, layer.topk_idx,
                                                layer.kept_idx, layer.group_dropped,
                                                layer.workspace)),
        ("moe_router_zloss", lambda: L.moe_router_zloss(dm, layer.logits, G, layer.group_z,
                                                        layer.workspace)),
        ("moe_permute", lambda: L.moe_permute(dm, table, layer.expert_counts,
                                              layer.expert_offsets, layer.pos, layer.src_token,
                                              x, layer.x_perm, layer.workspace)),
        ("moe_expert_up", lambda: L.moe_expert_up(dm, layer.x_perm, layer.expert_offsets, w1, w3,
                                                  layer.a, layer.b, layer.h)),
        # gathered expert input: the same two steps without x_perm
        ("moe_permute_plan", lambda: L.moe_permute(dm, table, layer.expert_counts,
                                                   layer.expert_offsets, layer.pos,
                                                   layer.src_token, None, None,
                                                   layer.workspace)),
        ("moe_expert_up_gather", lambda: L.moe_expert_up_gather(
            dm, x, layer.src_token, layer.expert_offsets, w1, w3, layer.a, layer.b, layer.h)),
        ("moe_expert_down", lambda: L.moe_expert_down(dm, layer.h, layer.expert_offsets, w2,
                                                      layer.y_perm)),
        ("moe_combine", lambda: L.moe_combine(dm, layer.y_perm, layer.pos,
                                              None if fold else layer.topk_gate, layer.y)),
        ("moe_combine_bwd", lambda: L.moe_combine_bwd(dm, dy, layer.y_perm, layer.pos,
                                                      layer.topk_gate, layer.dy_perm,
                                                      layer.dgate)),
        ("moe_expert_dgrad_down", lambda: L.moe_expert_dgrad_down(
            dm, layer.dy_perm, layer.expert_offsets, w2, layer.a, layer.b, da, db)),
        ("moe_expert_dgrad_up", lambda: L.moe_expert_dgrad_up(
            dm, da, db, layer.expert_offsets, w1, w3, layer.dx_perm)),
        ("moe_expert_wgrad", lambda: L.moe_expert_wgrad(
            dm, layer.x_perm, layer.expert_offsets, layer.h, layer.dy_perm, da, db, layer.dw1,
            layer.dw3, layer.dw2, layer.workspace)),
        ("moe_expert_wgrad_gather", lambda: L.moe_expert_wgrad_gather(
            dm, x, layer.src_token, layer.expert_offsets, layer.h, layer.dy_perm, da, db,
            layer.dw1, layer.dw3, layer.dw2, layer.workspace)),
        ("moe_route_bwd", lambda: L.moe_route_bwd(dm, x, wr, layer.topk_idx, layer.topk_gate,
                                                  layer.dgate, layer.expert_offsets, layer.pos,
                                                  layer.src_token, layer.dx_perm, layer.dx,
                                                  layer.dwr, layer.workspace)),
        ("moe_route_bwd_dense", lambda: L.moe_route_bwd_dense(
            dm, x, wr, layer.logits, layer.topk_idx, layer.topk_gate, layer.dgate, layer.pos,
            layer.dx_perm, G, layer.group_count, layer.aux_coef, layer.z_coef, layer.dx,
            layer.dwr, None, layer.workspace)),
    ]
    if fold:
        calls += [
            ("moe_permute_gates", lambda: L.moe_permute_gates(
                dm, table, layer.topk_gate, layer.expert_counts, layer.expert_offsets, layer.pos,
                layer.src_token, layer.gate_perm, layer.workspace)),
            ("moe_expert_up_folded", lambda: L.moe_expert_up_folded(
                dm, x, layer.src_token, layer.expert_offsets, layer.gate_perm, w1, w3, layer.a,
                layer.b, layer.h)),
            ("moe_expert_dgrad_down_folded", lambda: L.moe_expert_dgrad_down_folded(
                dm, dy, layer.src_token, layer.expert_offsets, layer.gate_perm, w2, layer.a,
                layer.b, da, db, layer.dgate_part)),
            ("moe_dgate_from_parts", lambda: L.moe_dgate_from_parts(
                dm, layer.dgate_part, layer.pos, layer.dgate)),
            ("moe_route_bwd_folded", lambda: L.moe_route_bwd_folded(
                dm, x, wr, layer.topk_idx, layer.topk_gate, layer.dgate_part,
                layer.expert_offsets, layer.pos, layer.src_token, layer.dx_perm, layer.dgate,
                layer.dx, layer.dwr, layer.workspace)),
            ("moe_expert_wgrad_folded", lambda: L.moe_expert_wgrad_folded(
                dm, x, dy, layer.src_token, layer.expert_offsets, layer.h, da, db, layer.dw1,
                layer.dw3, layer.dw2)),
        ]
        order = ["moe_route", "moe_capacity", "moe_router_zloss", "moe_permute_gates",
                 "moe_expert_up_folded", "moe_expert_down", "moe_combine",
                 "moe_expert_dgrad_down_folded", "moe_dgate_from_parts", "moe_expert_dgrad_up",
                 "moe_expert_wgrad_folded", "moe_route_bwd_folded", "moe_route_bwd_dense"]
        if layer.dense_bwd or L.moe_dgate_parts(dm) > 2:
            # the parts are summed once first (more than two per row would be
            # reloaded by every dX thread of the router backward)
            order.remove("moe_route_bwd_folded")
            if not layer.dense_bwd:
                order.insert(order.index("moe_route_bwd_dense"), "moe_route_bwd")
        else:   # the sparse router backward sums the dgate parts itself
            order.remove("moe_dgate_from_parts")
        by_name = dict(calls)
        calls = [(n, by_name[n]) for n in order]
    drop = (("moe_permute", "moe_expert_up", "moe_expert_wgrad") if gather else
            ("moe_permute_plan", "moe_expert_up_gather", "moe_expert_wgrad_gather"))
    drop += ("moe_route_bwd",) if layer.dense_bwd else ("moe_route_bwd_dense",)
    if layer.capacity is None:
        drop += ("moe_capacity",)
    if layer.z_coef == 0.0:
        drop += ("moe_router_zloss",)
    calls = [c for c in calls if c[0] not in drop]
    if not cfg.backward:
        calls = calls[:[c[0] for c in calls].index("moe_combine") + 1]

    if args.copy_calibration_mb > 0:
        nbytes = args.copy_calibration_mb << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()

    def eager_step():
        for _, fn in calls:
            fn()

    step = eager_step
    if args.graph:
        # one step captured in a HIP graph (the library allocates, frees and
        # synchronises nothing, and launches on torch's current stream, which
        # is the capture stream here); the timed region replays it
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            eager_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            eager_step()
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        step = graph.replay

    # Timed region (bracketed by synchronisations): K steps, each timed by its
    # own pair of events on the stream the library launches on (torch's
    # current stream).  Before each step a write of --flush-mb MiB evicts L2
    # and the MALL, outside the step's events: the headline is the median of
    # these cold-cache steps.  A second pass times K steps back to back with
    # warm caches (the median again).
    flush = (torch.empty(args.flush_mb << 18, dtype=torch.float32, device=dev)
             if args.flush_mb > 0 else None)

    def timed_steps(cold):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            if cold:
                flush.fill_(1.0)
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    cold_ms = timed_steps(True) if flush is not None else None
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    warm_ms = timed_steps(False)
    ms_per_step = float(np.median(cold_ms if cold_ms is not None else warm_ms))

    # Per-call durations (same stream, events around each call) in a third
    # pass of K warm steps; they carry the roofline and the breakdown.
    n = len(calls)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)] for _ in range(args.steps)]
    for s_ in range(args.steps):
        for i, (_, fn) in enumerate(calls):
            evs[s_][i][0].record()
            fn()
            evs[s_][i][1].record()
    torch.cuda.synchronize()
    per_call = {name: float(np.mean([evs[s_][i][0].elapsed_time(evs[s_][i][1])
                                     for s_ in range(args.steps)]))
                for i, (name, _) in enumerate(calls)}

    rows = int(layer.expert_offsets[cfg.E].item())   # expert rows (fewer when dropping)
    work = algorithmic_work(cfg, rows, fold, L.moe_dgate_parts(dm))
    # the dominant single-kernel call carries the roofline
    single = {n: t for n, t in per_call.items() if work[n][2] == 1 or
              (n in WGRAD_CALLS and wgrad_kernels(dm) == 1)}
    dominant = max(single, key=single.get)
    fl, by, _ = work[dominant]
    roof = roofline_entry(fl, by, per_call[dominant] * 1e-3, cfg.act)
    roof.update({"kernel": dominant, "traffic": measured_traffic(cfg.name, dominant)})
    gemm_ms = sum(per_call[n] for n in GEMM_CALLS if n in per_call)
    gemm_flops = sum(work[n][0] for n in GEMM_CALLS if n in per_call)
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "timing": {"statistic": "median over the timed steps",
                   "cold_cache": (f"{args.flush_mb} MiB written before every step, outside its "
                                  "events" if cold_ms is not None else None),
                   "ms_per_step_cold": (round(float(np.median(cold_ms)), 4)
                                        if cold_ms is not None else None),
                   "ms_per_step_warm": round(float(np.median(warm_ms)), 4),
                   "tokens_per_s_warm": round(cfg.T / (float(np.median(warm_ms)) * 1e-3), 1)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act,
        "data": "synthetic (seeded generators; random-init weights)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f} k={cfg.k} "
                               f"{cfg.act}, fp32 router, {'fwd+bwd' if cfg.backward else 'fwd'}",
                   "tokens": cfg.T, "lb_groups": G,
                   "expert_input": "gathered from X by src_token" if gather
                                   else "materialised x_perm",
                   "gate": "folded onto the expert rows" if fold else "applied in the combine",
                   "launch": "HIP graph replay" if args.graph else "eager launches"},
        "grouped_gemm": {"tflops": round(gemm_tflops, 2),
                         "frac_of_peak": round(gemm_tflops / (PEAK_MFMA[cfg.act] / 1e12), 4)},
        "per_call_ms": {k: round(v, 4) for k, v in per_call.items()},
        "wall_s": round(wall, 3),
        "roofline": roof,
        # every call against its own bound (algorithmic work over its mean duration)
        "per_call_roofline": {
            n: {k2: v2 for k2, v2 in roofline_entry(work[n][0], work[n][1], t * 1e-3,
                                                     cfg.act).items() if k2 in ("bound", "frac")}
            for n, t in per_call.items()},
    }
    if layer.dense_bwd:
        out["config"]["variant"] = {
            "capacity_factor": args.capacity_factor, "capacity": layer.capacity,
            "aux_coef": layer.aux_coef, "z_coef": layer.z_coef, "expert_rows": rows,
            "dropped": (int(layer.group_dropped.sum().item())
                        if layer.group_dropped is not None else 0)}
    if args.ep and cfg.plan_groups:
        out["ep_dispatch"] = ep_dispatch(cfg, layer, x, wr, args.steps)
    if args.fragility:
        out["fragility"] = fragility(cfg, layer, x, wr, args.steps)
    if args.shuffle and cfg.plan_groups:
        out["token_shuffle"] = token_shuffle(cfg, layer, x, wr, args.steps)
    if not args.no_reports:
        out["reports"] = workload_reports(args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
