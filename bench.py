"""Benchmark: MoE layer forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

One step is one full pass of the layer's hot path over one batch of synthetic
tokens: moe_route -> moe_permute -> moe_grouped_swiglu_fwd -> moe_combine ->
moe_combine_bwd -> moe_grouped_swiglu_bwd -> moe_route_bwd.  Inputs and weights
are resident in HBM before timing starts.  Prints one JSON line.

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


def algorithmic_work(cfg):
    """Per-call algorithmic (flops, bytes): what each call must compute and move
    (inputs read once, outputs written once, as its C-ABI contract states)."""
    T, d, E, f, k = cfg.T, cfg.d, cfg.E, cfg.f, cfg.k
    R = T * k
    s = 2 if cfg.act == "bf16" else 4
    i4 = 4
    W = 3 * E * d * f * s
    return {
        "moe_route": (2 * T * d * E,
                      T * d * s + E * d * 4 + T * E * 4 + T * k * (i4 + 4) + T * 4),
        "moe_permute": (0, T * k * i4 + T * d * s + R * d * s + 2 * R * i4 + (2 * E + 1) * i4),
        "moe_grouped_swiglu_fwd": (6 * R * d * f, R * d * s + W + 3 * R * f * s + R * d * s),
        "moe_combine": (2 * R * d, R * d * s + T * d * s + T * k * (i4 + 4)),
        "moe_combine_bwd": (2 * R * d, T * d * s + 2 * R * d * s + T * k * (i4 + 8)),
        "moe_grouped_swiglu_bwd": (12 * R * d * f,
                                   2 * R * d * s + 3 * R * f * s + W + R * d * s + W),
        "moe_route_bwd": (4 * R * d, T * d * s + E * d * 4 + R * d * s + T * d * s + E * d * 4
                          + T * k * 12 + R * 8),
    }


def roofline_entry(flops, nbytes, seconds, act):
    peak_f = PEAK_MFMA[act]
    if flops / peak_f > nbytes / PEAK_HBM:
        achieved = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_f / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / (peak_f / 1e12), 4)}
    achieved = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
            "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4)}


def cpu_baseline(cfg, inp, budget_s=20.0):
    """The oracle as it stands (fp64 numpy), on the same workload, timed on the
    host cores.  Runs whole steps of the full workload until budget_s is spent
    (at least one)."""
    import threadpoolctl
    from oracle import moe_oracle as O
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    steps = 0
    while True:
        fwd = O.layer_forward(inp["x"], inp["wr"], inp["w1"], inp["w3"], inp["w2"], cfg.k)
        if cfg.backward:
            O.layer_backward(inp["x"], inp["wr"], inp["w1"], inp["w3"], inp["w2"], fwd, inp["dy"])
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (steps + 1) / steps > 3 * budget_s:
            break
    return {"value": round(cfg.T * steps / el, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} full step(s) of {cfg.name} ({cfg.T} tokens, fwd"
                      f"{'+bwd' if cfg.backward else ''}), fp64 numpy, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of tokens; --gpus {args.gpus} is not "
              "supported (this build runs on a single GPU).", file=sys.stderr)
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
    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=G)
    dm = layer.dims

    calls = [
        ("moe_route", lambda: layer.route(x, wr)),
        ("moe_permute", lambda: L.moe_permute(dm, layer.topk_idx, layer.expert_counts,
                                              layer.expert_offsets, layer.pos, layer.src_token,
                                              x, layer.x_perm, layer.workspace)),
        ("moe_grouped_swiglu_fwd", lambda: L.moe_grouped_swiglu_fwd(
            dm, layer.x_perm, layer.expert_offsets, w1, w3, w2, layer.a, layer.b, layer.h,
            layer.y_perm)),
        ("moe_combine", lambda: L.moe_combine(dm, layer.y_perm, layer.pos, layer.topk_gate,
                                              layer.y)),
        ("moe_combine_bwd", lambda: L.moe_combine_bwd(dm, dy, layer.y_perm, layer.pos,
                                                      layer.topk_gate, layer.dy_perm,
                                                      layer.dgate)),
        ("moe_grouped_swiglu_bwd", lambda: L.moe_grouped_swiglu_bwd(
            dm, layer.x_perm, layer.expert_offsets, w1, w3, w2, layer.a, layer.b, layer.h,
            layer.dy_perm, layer.dx_perm, layer.dw1, layer.dw3, layer.dw2, layer.workspace)),
        ("moe_route_bwd", lambda: L.moe_route_bwd(dm, x, wr, layer.topk_idx, layer.topk_gate,
                                                  layer.dgate, layer.expert_offsets, layer.pos,
                                                  layer.src_token, layer.dx_perm, layer.dx,
                                                  layer.dwr, layer.workspace)),
    ]
    if not cfg.backward:
        calls = calls[:4]

    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()

    n = len(calls)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        for i, (_, fn) in enumerate(calls):
            evs[s][i][0].record()
            fn()
            evs[s][i][1].record()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    per_call = {name: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1])
                                     for s in range(args.steps)]))
                for i, (name, _) in enumerate(calls)}

    work = algorithmic_work(cfg)
    dominant = max(per_call, key=per_call.get)
    fl, by = work[dominant]
    roof = roofline_entry(fl, by, per_call[dominant] * 1e-3, cfg.act)
    roof.update({"kernel": dominant, "traffic": None})
    gemm_ms = per_call["moe_grouped_swiglu_fwd"] + per_call.get("moe_grouped_swiglu_bwd", 0.0)
    gemm_flops = work["moe_grouped_swiglu_fwd"][0] + (
        work["moe_grouped_swiglu_bwd"][0] if cfg.backward else 0)
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act,
        "data": "synthetic (seeded generators; random-init weights)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f} k={cfg.k} "
                               f"{cfg.act}, fp32 router, {'fwd+bwd' if cfg.backward else 'fwd'}",
                   "tokens": cfg.T, "lb_groups": G},
        "grouped_gemm": {"tflops": round(gemm_tflops, 2),
                         "frac_of_peak": round(gemm_tflops / (PEAK_MFMA[cfg.act] / 1e12), 4)},
        "per_call_ms": {k: round(v, 4) for k, v in per_call.items()},
        "wall_s": round(wall, 3),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
