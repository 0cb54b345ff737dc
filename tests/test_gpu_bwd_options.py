"""GPU: the two options of the expert backward call (moe_grouped_swiglu_bwd
and its gathered form).

* wgrad_dtype = fp32 on a bf16 layer.  dW1, dW3 and dW2 are held to the
  exact fp64 oracle within C_BOUND times their first-order bound (its storage
  term is that of bf16, so it also covers the smaller fp32 rounding), every
  other output to the same rules as the default layer; the weight gradients
  must really be fp32 (nearly all of them off the bf16 grid); and where the
  bf16 call runs the same split-K kernels (few output tiles), rounding the
  fp32 weight gradients to bf16 gives the bf16 call's bits.
* a_save = b_save = h_save = NULL.  The call recomputes a, b and h with the
  forward kernel from the expert input; every output equals that of the call
  given the saved activations, bit for bit, for bf16 and fp32 layers, with
  x_perm and with the gathered input, with either weight-gradient type.

Shapes reach the weight-gradient stream with fp32 output both through the
split-K reduction (ragged, few tiles) and straight from the accumulators
(C2's width at full size, 256 experts), and the forward kernels that the
recomputation runs (persistent small tile, big direct-to-LDS tile, fp32).
"""
import ctypes

import numpy as np
import pytest
import torch

from synth import get_config, make_layer_inputs, stream
import top_routing_grouped_router_amd._lib as L
from top_routing_grouped_router_amd import MoELayer

from _parity import (bound_only_keys, check_plan, check_route, exact_reference, layer_floats,
                     oracle_routing)
from _util import TOL, act_torch, check_floats, dev, host

pytestmark = pytest.mark.gpu

WGRAD_CASES = {
    # name: (T, d, E, f, k)   -- bf16 layers
    "ragged_split_k": (1000, 256, 8, 192, 3),
    "c2_width_full": (16384, 256, 16, 256, 4),
    "max_experts": (260, 64, 256, 64, 16),
}


def _layer(cfg, inp, routing, **kw):
    act = act_torch(cfg.act)
    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, **kw)
    t = {k: dev(v, act) for k, v in inp.items() if k != "wr"}
    t["wr"] = dev(inp["wr"], torch.float32)
    layer.forward(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], routing=routing)
    layer.backward(t["dy"], t["x"], t["wr"], t["w1"], t["w3"], t["w2"])
    torch.cuda.synchronize()
    return layer


def _print_cancellation(name, o_f, o_b):
    """Median over rows of max_j sum|terms| / max_j |sum| for dW1 and dW3
    (the size of the summed terms against the size of the result)."""
    off, xp = o_f["offsets"], np.abs(o_f["x_perm"])
    for key, op in (("dw1", "da"), ("dw3", "db")):
        ratios = []
        for e in range(len(off) - 1):
            s = slice(int(off[e]), int(off[e + 1]))
            if off[e + 1] == off[e]:
                continue
            terms = np.abs(o_b[op][s]).T @ xp[s]
            res = np.abs(o_b[key][e])
            ratios.append(terms.max(axis=1) / np.maximum(res.max(axis=1), 1e-300))
        print(f"[{name}] {key}: median row sum|terms| / |sum| = {np.median(np.concatenate(ratios)):.2f}",
              flush=True)


@pytest.mark.parametrize("name", list(WGRAD_CASES))
def test_fp32_weight_gradients_of_a_bf16_layer(name):
    print(f"\n[case] fp32 dW {name}", flush=True)
    T, d, E, f, k = WGRAD_CASES[name]
    cfg = get_config("c2", T=T, d=d, E=E, f=f, k=k, act="bf16", x_kind="normal",
                     backward=True)
    inp = make_layer_inputs(cfg, seed=300 + list(WGRAD_CASES).index(name))
    probe = MoELayer(T, d, E, f, k, torch.bfloat16)
    o_route, _ = check_route(probe, inp["x"], inp["wr"], k)
    routing = (o_route["topk_idx"], o_route["gates"].astype(np.float32))
    dmr = oracle_routing(o_route)
    wide = _layer(cfg, inp, dmr, wgrad_dtype=torch.float32)
    assert wide.dw1.dtype == torch.float32 and wide.dw2.dtype == torch.float32

    o_f, o_b, B = exact_reference(inp, k, routing, act="bf16")
    check_plan(wide, o_f)
    got, ex, bd = layer_floats(wide, o_f, o_b, B)
    bound_only = bound_only_keys(cfg)
    if T * k < 64 * E:
        # about 16 rows per expert: each weight-gradient entry sums a few
        # terms of random sign, so the bf16 storage of da, db and h upstream
        # (not the fp32 output) moves it by more than 2e-2 of its row in places
        bound_only += ("dw1", "dw3", "dw2")
        _print_cancellation(name, o_f, o_b)
    check_floats(f"{name} fp32 dW", got, ex, bd, TOL["bf16"], bound_only)

    narrow = _layer(cfg, inp, dmr)
    same_kernels = L.lib().moe_expert_wgrad_launches(ctypes.byref(narrow.dims)) == 2
    for key in ("dw1", "dw3", "dw2"):
        w = getattr(wide, key)
        nz = w != 0
        off_grid = (w != w.to(torch.bfloat16).float()) & nz
        frac = off_grid.sum().item() / max(nz.sum().item(), 1)
        assert frac > 0.9, f"{key}: only {frac:.3f} of the fp32 weight gradients are off the bf16 grid"
        if same_kernels:
            assert torch.equal(w.to(torch.bfloat16), getattr(narrow, key)), key
    # everything upstream of the weight gradients is the bf16 layer's, bit for bit
    for key in ("y", "dx_perm", "dgate", "dx", "dwr"):
        assert torch.equal(getattr(wide, key), getattr(narrow, key)), key


RECOMPUTE_CASES = {
    # name: (T, d, E, f, k, act)
    "ragged_bf16": (1000, 256, 8, 192, 3, "bf16"),
    "ragged_f32": (777, 128, 6, 128, 2, "f32"),
    "c2_shape": (16384, 256, 16, 256, 4, "bf16"),
    "big_tile": (8192, 1024, 16, 1024, 2, "bf16"),
    "max_experts": (260, 64, 256, 64, 16, "bf16"),
}


def _rand(rng, shape, ta, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(a).to("cuda", ta).contiguous()


@pytest.mark.parametrize("name", list(RECOMPUTE_CASES))
def test_recompute_matches_saved_activations(name):
    print(f"\n[case] recompute {name}", flush=True)
    T, d, E, f, k, act = RECOMPUTE_CASES[name]
    rng = stream(9, 200 + list(RECOMPUTE_CASES).index(name))
    ta = act_torch(act)
    layer = MoELayer(T, d, E, f, k, ta)
    dm = layer.dims
    x = _rand(rng, (T, d), ta)
    wr = _rand(rng, (E, d), torch.float32, d ** -0.5)
    w1, w3 = _rand(rng, (E, f, d), ta, d ** -0.5), _rand(rng, (E, f, d), ta, d ** -0.5)
    w2 = _rand(rng, (E, d, f), ta, f ** -0.5)
    dy = _rand(rng, (T * k, d), ta)
    layer.route(x, wr)
    L.moe_permute(dm, layer.topk_idx, layer.expert_counts, layer.expert_offsets, layer.pos,
                  layer.src_token, x, layer.x_perm, layer.workspace)
    R = T * k
    off, src = layer.expert_offsets, layer.src_token
    a, b, h = (torch.empty(R, f, device="cuda", dtype=ta) for _ in range(3))
    y = torch.empty(R, d, device="cuda", dtype=ta)
    L.moe_grouped_swiglu_fwd(dm, layer.x_perm, off, w1, w3, w2, a, b, h, y)
    ws = torch.empty(L.moe_grouped_swiglu_bwd_workspace_bytes(dm, True), dtype=torch.uint8,
                     device="cuda")
    wdts = (ta,) if act == "f32" else (ta, torch.float32)
    for wdt in wdts:
        outs = {}
        for mode in ("saved", "recompute", "saved_gather", "recompute_gather"):
            dx = torch.empty(R, d, device="cuda", dtype=ta)
            dws = [torch.empty(E, f, d, device="cuda", dtype=wdt),
                   torch.empty(E, f, d, device="cuda", dtype=wdt),
                   torch.empty(E, d, f, device="cuda", dtype=wdt)]
            saved = (None, None, None) if mode.startswith("recompute") else (a, b, h)
            if mode.endswith("gather"):
                L.moe_grouped_swiglu_bwd_gather(dm, x, src, off, w1, w3, w2, *saved, dy, dx,
                                                *dws, ws, wgrad_dtype=wdt)
            else:
                L.moe_grouped_swiglu_bwd(dm, layer.x_perm, off, w1, w3, w2, *saved, dy, dx,
                                         *dws, ws, wgrad_dtype=wdt)
            torch.cuda.synchronize()
            outs[mode] = (dx, *dws)
        ref = outs["saved"]
        for mode, o in outs.items():
            for u, v, key in zip(ref, o, ("dx_perm", "dw1", "dw3", "dw2")):
                assert torch.equal(u, v), f"{mode} {wdt} {key}"


def test_recompute_layer_step():
    """A whole layer step with recompute=True (materialised and gathered
    input) gives the default step's outputs bit for bit."""
    print("\n[case] recompute layer step", flush=True)
    T, d, E, f, k = 4096, 256, 16, 256, 4
    rng = stream(9, 1)
    x = _rand(rng, (T, d), torch.bfloat16)
    wr = _rand(rng, (E, d), torch.float32, d ** -0.5)
    w1 = _rand(rng, (E, f, d), torch.bfloat16, d ** -0.5)
    w3 = _rand(rng, (E, f, d), torch.bfloat16, d ** -0.5)
    w2 = _rand(rng, (E, d, f), torch.bfloat16, f ** -0.5)
    dy = _rand(rng, (T, d), torch.bfloat16)
    for gather in (False, True):
        ref = MoELayer(T, d, E, f, k, torch.bfloat16, gather=gather)
        ref.step(x, wr, w1, w3, w2, dy)
        rec = MoELayer(T, d, E, f, k, torch.bfloat16, gather=gather, recompute=True)
        rec.step(x, wr, w1, w3, w2, dy)
        torch.cuda.synchronize()
        for key in ("y", "dx", "dw1", "dw3", "dw2", "dwr"):
            assert torch.equal(getattr(ref, key), getattr(rec, key)), (gather, key)
