"""GPU: the gate-folded layer (gate moved onto the expert rows; dY read
through src_token, no dy_perm) against the EXACT fp64 oracle layer (gate in
the combine, nothing rounded), element by element within C_BOUND times the
first-order error bound, and within 2e-2 row-normwise outside the weight
gradients of clustered-input workloads.  The oracle's folded storage mode is
not used as a reference: the folded and unfolded GPU layers are held to the
same exact values.

The oracle's routing and block counts are copied into the layer, so integer
outputs compare bit for bit.  Cases: C2 and C3 at full size (the 8- and
4-stage weight-gradient rings), a ragged shape whose f = 192 leaves a partial
column tile for the dgate parts, C2 with capacity and both losses (dropped
slots, dense router backward), a shape whose UP, dgrad_down and weight
gradients all take the big tile, and the same with f = 1152, whose last
256-wide dgate-part column tile is half empty.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import get_config, make_layer_inputs
from top_routing_grouped_router_amd import MoELayer
import top_routing_grouped_router_amd._lib as L

from _parity import bound_only_keys, exact_reference, layer_floats
from _util import TOL, act_torch, check_floats, dev, host, rel_err

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, overrides, G, capacity factor, aux_coef, z_coef)
    "c2": ("c2", {}, 8, None, 0.0, 0.0),
    "c3": ("c3", {}, 8, None, 0.0, 0.0),
    "ragged_f192": ("c2", dict(T=1000, d=256, E=16, f=192, k=3), 4, None, 0.0, 0.0),
    "c2_cap1_losses": ("c2", dict(T=4096), 4, 1.0, 0.01, 0.001),
    # UP, dgrad_down and the weight gradients on the 256 x 256 tile
    "big_tiles": ("c5", dict(T=8192, d=1024, E=16, f=1024, k=4), 4, None, 0.0, 0.0),
    # the same with a partial last 256-wide column tile of f (1152 = 4.5 x 256)
    "big_tiles_f1152": ("c5", dict(T=8192, d=1024, E=16, f=1152, k=4), 4, None, 0.0, 0.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_folded_layer_matches_oracle(name):
    base, over, G, factor, aux_coef, z_coef = CASES[name]
    print(f"\n[case] folded {name}", flush=True)
    cfg = get_config(base, **over)
    inp = make_layer_inputs(cfg, seed=23, with_dy=True)
    act = act_torch(cfg.act)
    C = None if factor is None else O.expert_capacity(cfg.T, cfg.k, cfg.E, G, factor)
    r = O.route(inp["x"], inp["wr"], cfg.k)
    routing = (r["topk_idx"], r["gates"].astype(np.float32))
    o_f, o_b, B = exact_reference(inp, cfg.k, routing, act=cfg.act, capacity=C, lb_groups=G,
                                  aux_coef=aux_coef, z_coef=z_coef)
    count = O.lb_stats(o_f["logits"], o_f["topk_idx"], cfg.E, G)["count"]

    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=G, gather=True,
                     capacity_factor=factor, aux_coef=aux_coef, z_coef=z_coef, fold_gate=True)
    t = {key: dev(v, act) for key, v in inp.items() if key != "wr"}
    t["wr"] = dev(inp["wr"], torch.float32)
    layer.route(t["x"], t["wr"])
    layer.topk_idx.copy_(dev(o_f["topk_idx"], torch.int32))
    layer.topk_gate.copy_(dev(routing[1], torch.float32))
    layer.group_count.copy_(dev(count, torch.int32))
    layer.forward_experts(t["x"], t["w1"], t["w3"], t["w2"])
    layer.backward(t["dy"], t["x"], t["wr"], t["w1"], t["w3"], t["w2"])
    torch.cuda.synchronize()

    R = int(o_f["offsets"][-1])
    kept = o_f["kept_idx"] if C is not None else o_f["topk_idx"]
    assert np.array_equal(host(layer.expert_offsets), o_f["offsets"])
    assert np.array_equal(host(layer.pos), o_f["pos"])
    assert np.array_equal(host(layer.src_token)[:R], o_f["src"][:R])
    got, ex, bd = layer_floats(layer, o_f, o_b, B)
    check_floats(f"folded {name}", got, ex, bd, TOL["bf16"], bound_only_keys(cfg))
    if C is not None:
        assert o_f["dropped"].sum() > 0
        assert np.all(host(layer.dgate)[kept < 0] == 0.0)


def test_folded_matches_unfolded_layer():
    """Same inputs, same routing (the router runs in both): integer outputs
    equal, floats a rounding step apart."""
    print("\n[case] folded vs unfolded c2 T=4096", flush=True)
    cfg = get_config("c2", T=4096)
    inp = make_layer_inputs(cfg, seed=29, with_dy=True)
    act = act_torch(cfg.act)
    t = {key: dev(v, act) for key, v in inp.items() if key != "wr"}
    t["wr"] = dev(inp["wr"], torch.float32)
    a = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=4, gather=True)
    b = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=4, gather=True,
                 fold_gate=True)
    for layer in (a, b):
        layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])
    torch.cuda.synchronize()
    for key in ("topk_idx", "pos", "src_token", "expert_offsets", "group_count"):
        assert np.array_equal(host(getattr(a, key)), host(getattr(b, key))), key
    for key in ("y", "dgate", "dx", "dw1", "dw3", "dw2", "dwr"):
        e = rel_err(host(getattr(b, key)), host(getattr(a, key)))
        print(f"[folded vs unfolded] {key} {e:.1e}", flush=True)
        assert e <= TOL["bf16"], (key, e)


def test_folded_calls_reject_unsupported_dims():
    cfg = get_config("c2", T=1000, d=256, E=8, f=192, k=3)   # split-K weight gradients
    dims = L.make_dims(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, torch.bfloat16)
    assert not L.moe_gate_folded_supported(dims)
    z = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    zi = torch.empty(16, dtype=torch.int32, device="cuda")
    zf = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(L.MoEError):
        L.moe_expert_up_folded(dims, z, zi, zi, zf, z, z, z, z, z)
    with pytest.raises(ValueError):
        MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, torch.bfloat16, gather=True, fold_gate=True)


def test_folded_layer_on_an_empty_batch():
    """T = 0: every folded call runs, the weight gradients are zero."""
    print("\n[case] folded T=0", flush=True)
    T, d, E, f, k = 0, 256, 16, 256, 4
    layer = MoELayer(T, d, E, f, k, torch.bfloat16, n_groups=1, gather=True, fold_gate=True)
    x = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    wr = torch.randn((E, d), device="cuda")
    w1 = torch.randn((E, f, d), device="cuda").to(torch.bfloat16)
    w3 = torch.randn((E, f, d), device="cuda").to(torch.bfloat16)
    w2 = torch.randn((E, d, f), device="cuda").to(torch.bfloat16)
    for name in ("dw1", "dw3", "dw2", "dwr"):
        getattr(layer, name).fill_(float("nan"))
    layer.step(x, wr, w1, w3, w2, dy)
    torch.cuda.synchronize()
    for name in ("dw1", "dw3", "dw2", "dwr"):
        assert torch.all(getattr(layer, name) == 0), name
    assert int(layer.expert_offsets[E].item()) == 0
