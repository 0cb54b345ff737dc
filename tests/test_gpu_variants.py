"""GPU parity of the definitional variants against the oracle: per-block expert
capacity with dropping (moe_capacity), the router z-loss values
(moe_router_zloss) and the dense router backward that carries dropped slots
and the balancing and z-loss gradients (moe_route_bwd_dense), alone and inside
a whole layer step.

Rules: kept tables, dropped counts, counts, offsets, positions and source
tokens bit-exact; router quantities (z-loss values, the logit gradient when
the upstream gradients are exact) within 1e-4; in the whole-layer cases every
float output is held to the exact fp64 oracle layer (C_BOUND times its
first-order error bound, and the workload's tolerance, 1e-4 fp32 or 2e-2 bf16,
row-normwise), on the oracle's routing uploaded to the GPU.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import get_config, make_layer_inputs, make_routing, stream
from synth.generate import bf16_round
from top_routing_grouped_router_amd import MoELayer
import top_routing_grouped_router_amd as M

from _parity import bound_only_keys, exact_reference, layer_floats
from _util import TOL, TOL_ROUTER, act_torch, check_floats, dev, host, per_slice_err, rel_err

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"\n[case] {name}", flush=True)


# ---------------------------------------------------------------- capacity kernel

CAP_CASES = [
    # (T, E, k, G, factor)
    (96, 8, 3, 1, 1.0),           # one chunk
    (4096, 16, 4, 1, 1.0),        # 16 chunks in one block
    (4096, 16, 4, 8, 1.25),
    (2048, 64, 6, 4, 0.5),
    (1000, 256, 16, 8, 2.0),      # largest E and k; ragged last chunk
    (777, 5, 2, 7, 1.0),
    (512, 8, 2, 2, 0.0),          # capacity 0: everything dropped
    (512, 8, 2, 2, 100.0),        # nothing dropped
    (16384, 64, 6, 8, 1.0),       # full-size shape (16384 tokens, 64 experts, top-6)
]


@pytest.mark.parametrize("case", CAP_CASES)
def test_capacity_kernel_bit_exact(case):
    T, E, k, G, factor = case
    _announce(f"capacity T={T} E={E} k={k} G={G} factor={factor}")
    # skewed routing so that capacity binds on the popular experts
    g = stream(61, T + E)
    logits = g.standard_normal((T, E)) + np.linspace(2.0, 0.0, E)[None, :]
    idx, _ = O.topk_select(logits, k)
    C = M.moe_expert_capacity(T, k, E, G, factor)
    assert C == O.expert_capacity(T, k, E, G, factor)
    ref = O.capacity_keep(idx, E, G, C)
    dims = M.make_dims(T, 64, E, 64, k, torch.bfloat16)
    kept = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    dropped = torch.full((G,), -7, dtype=torch.int32, device="cuda")
    M.moe_capacity(dims, G, C, dev(idx, torch.int32), kept, dropped, M.alloc_workspace(dims, G))
    torch.cuda.synchronize()
    assert np.array_equal(host(kept), ref["kept_idx"])
    assert np.array_equal(host(dropped), ref["dropped"])


def test_capacity_then_permute_skips_dropped():
    _announce("capacity -> permute")
    T, E, k, G = 3000, 12, 3, 6
    idx = make_routing(T, E, k, seed=5)
    C = O.expert_capacity(T, k, E, G, 0.8)
    ref = O.capacity_keep(idx, E, G, C)
    plan = O.permute_plan(ref["kept_idx"], E)
    R = int(plan["offsets"][-1])
    assert 0 < R < T * k
    dims = M.make_dims(T, 128, E, 64, k, torch.bfloat16)
    kept = torch.empty((T, k), dtype=torch.int32, device="cuda")
    dropped = torch.empty((G,), dtype=torch.int32, device="cuda")
    ws = M.alloc_workspace(dims, G)
    M.moe_capacity(dims, G, C, dev(idx, torch.int32), kept, dropped, ws)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
    x = dev(stream(5, 1).standard_normal((T, 128)).astype(np.float32), torch.bfloat16)
    x_perm = torch.zeros((T * k, 128), dtype=torch.bfloat16, device="cuda")
    M.moe_permute(dims, kept, counts, offsets, pos, src, x, x_perm, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(counts), plan["counts"])
    assert np.array_equal(host(offsets), plan["offsets"])
    assert np.array_equal(host(pos), plan["pos"])
    assert np.array_equal(host(src)[:R], plan["src"][:R])
    assert np.array_equal(host(x_perm)[:R], host(x)[plan["src"][:R]])


def test_capacity_rejects_bad_arguments():
    dims = M.make_dims(64, 64, 8, 64, 2, torch.bfloat16)
    idx = torch.zeros((64, 2), dtype=torch.int32, device="cuda")
    kept = torch.empty_like(idx)
    dropped = torch.empty(4, dtype=torch.int32, device="cuda")
    ws = M.alloc_workspace(dims, 4)
    with pytest.raises(M.MoEError):
        M.moe_capacity(dims, 3, 4, idx, kept, dropped, ws)      # 3 does not divide 64
    with pytest.raises(M.MoEError):
        M.moe_capacity(dims, 4, -1, idx, kept, dropped, ws)     # negative capacity
    with pytest.raises(M.MoEError):
        M.moe_capacity(dims, 4, 4, idx, kept, dropped, ws[:8])  # workspace too small
    with pytest.raises(M.MoEError):
        M.moe_expert_capacity(64, 2, 8, 3, 1.0)
    with pytest.raises(M.MoEError):
        M.moe_expert_capacity(64, 2, 8, 4, float("nan"))


# ---------------------------------------------------------------- z-loss values

@pytest.mark.parametrize("T,E,G", [(1000, 8, 4), (16384, 64, 8), (300, 256, 3), (0, 16, 1)])
def test_router_zloss_values(T, E, G):
    _announce(f"zloss T={T} E={E} G={G}")
    logits = (3.0 * stream(62, E).standard_normal((T, E))).astype(np.float32)
    dims = M.make_dims(T, 64, E, 64, 1, torch.float32)
    gz = torch.full((G,), float("nan"), dtype=torch.float32, device="cuda")
    lg = dev(logits, torch.float32) if T else torch.empty((1, E), device="cuda")[:0]
    M.moe_router_zloss(dims, lg, G, gz, M.alloc_workspace(dims, G))
    torch.cuda.synchronize()
    if T == 0:
        assert np.all(host(gz) == 0.0)
        return
    assert rel_err(host(gz), O.z_loss_groups(logits, G)) <= TOL_ROUTER


# ---------------------------------------------------------------- dense router backward

DENSE_CASES = [
    # (T, d, E, k, G, act, factor, aux_coef, z_coef)
    (1000, 256, 8, 3, 4, "bf16", 1.0, 0.1, 0.01),
    (777, 128, 6, 2, 7, "f32", 0.75, 0.3, 0.2),
    (260, 64, 256, 16, 4, "bf16", 1.0, 0.05, 0.01),   # E > 128: four experts per lane
    (300, 64, 100, 5, 3, "f32", None, 0.2, 0.0),       # E not a multiple of 16; aux only
    (512, 192, 16, 4, 2, "bf16", None, 0.0, 0.05),     # z only; d not a multiple of 256
    (16384, 2048, 64, 6, 8, "bf16", 1.0, 0.01, 0.001),  # full-size shape, launch as in the bench
]


@pytest.mark.parametrize("case", DENSE_CASES)
def test_route_bwd_dense_entry_point(case):
    T, d, E, k, G, act_name, factor, aux_coef, z_coef = case
    _announce(f"route_bwd_dense T={T} d={d} E={E} k={k} G={G} {act_name} cap={factor} "
              f"aux={aux_coef} z={z_coef}")
    act = act_torch(act_name)
    g = stream(63, T + d + E)
    x = g.standard_normal((T, d)).astype(np.float32)
    if act_name == "bf16":
        x = bf16_round(x)
    wr = (g.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    logits = (2.0 * g.standard_normal((T, E))).astype(np.float32)
    idx, _ = O.topk_select(logits, k)
    gates = O.chosen_gates(logits, idx).astype(np.float32)
    dgate = g.standard_normal((T, k)).astype(np.float32)
    kept = idx
    if factor is not None:
        kept = O.capacity_keep(idx, E, G, O.expert_capacity(T, k, E, G, factor))["kept_idx"]
        dgate = np.where(kept >= 0, dgate, 0.0).astype(np.float32)
    plan = O.permute_plan(kept, E)
    R = T * k
    dx_perm = g.standard_normal((R, d)).astype(np.float32)
    if act_name == "bf16":
        dx_perm = bf16_round(dx_perm)
    count = O.lb_stats(logits, idx, E, G)["count"]
    ref = O.route_bwd(x, wr, idx, gates, dgate, logits, count, aux_coef, z_coef)
    dx_ref = O.combine(dx_perm, plan["pos"], None) + ref["dx_router"]

    dims = M.make_dims(T, d, E, 64, k, act)
    dx = torch.empty((T, d), dtype=act, device="cuda")
    dwr = torch.empty((E, d), dtype=torch.float32, device="cuda")
    dl = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = M.alloc_workspace(dims, G)
    M.moe_route_bwd_dense(dims, dev(x, act), dev(wr, torch.float32), dev(logits, torch.float32),
                          dev(idx, torch.int32), dev(gates, torch.float32),
                          dev(dgate, torch.float32), dev(plan["pos"], torch.int32),
                          dev(dx_perm, act), G, dev(count, torch.int32), aux_coef, z_coef, dx,
                          dwr, dl, ws)
    torch.cuda.synchronize()
    e_dl = rel_err(host(dl), ref["dlogits"])
    e_dx = rel_err(host(dx), dx_ref)
    e_dwr = per_slice_err(host(dwr), ref["dwr"])
    print(f"[errors] dlogits {e_dl:.2e} dx {e_dx:.2e} dwr {e_dwr:.2e}", flush=True)
    assert e_dl <= TOL_ROUTER
    assert e_dx <= (TOL_ROUTER if act_name == "f32" else TOL["bf16"])
    assert e_dwr <= TOL_ROUTER


def test_route_bwd_dense_equals_sparse_without_variants():
    """No drops, zero coefficients: the dense form gives the sparse form's
    results up to summation order."""
    _announce("dense == sparse")
    cfg = get_config("c2", T=2048)
    inp = make_layer_inputs(cfg, seed=3, with_dy=True)
    act = act_torch(cfg.act)
    t = {key: dev(v, act) for key, v in inp.items() if key != "wr"}
    t["wr"] = dev(inp["wr"], torch.float32)
    G = 4
    a = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=G)
    b = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=G)
    b.dense_bwd = True
    b.dlogits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    for layer in (a, b):
        layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])
    torch.cuda.synchronize()
    assert np.array_equal(host(a.dgate), host(b.dgate))
    assert rel_err(host(b.dwr), host(a.dwr)) <= 1e-5
    assert rel_err(host(b.dx), host(a.dx)) <= 1e-2     # bf16 outputs: a rounding step apart
    assert np.mean(host(b.dx) != host(a.dx)) < 0.01


# ---------------------------------------------------------------- whole layer step

LAYER_CASES = {
    # name: (config, overrides, G, capacity factor, aux_coef, z_coef, gather)
    "ragged_bf16_cap1": ("c2", dict(T=1000, d=256, E=8, f=192, k=3, x_kind="normal"), 4, 1.0,
                         0.1, 0.01, True),
    "ragged_f32_cap075": ("c2", dict(T=777, d=128, E=6, f=128, k=2, act="f32",
                                     x_kind="normal"), 7, 0.75, 0.3, 0.2, False),
    "c2_cap1_losses": ("c2", {}, 8, 1.0, 0.01, 0.001, True),
    "c3_cap125_losses": ("c3", {}, 8, 1.25, 0.01, 0.001, True),
}


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_layer_step_with_capacity_and_losses(name):
    base, over, G, factor, aux_coef, z_coef, gather = LAYER_CASES[name]
    _announce(f"layer {name}")
    cfg = get_config(base, backward=True, **over) if over else get_config(base)
    inp = make_layer_inputs(cfg, seed=17, with_dy=True)
    act = act_torch(cfg.act)
    C = O.expert_capacity(cfg.T, cfg.k, cfg.E, G, factor)
    r = O.route(inp["x"], inp["wr"], cfg.k)
    routing = (r["topk_idx"], r["gates"].astype(np.float32))
    o_f, o_b, B = exact_reference(inp, cfg.k, routing, act=cfg.act, capacity=C, lb_groups=G,
                                  aux_coef=aux_coef, z_coef=z_coef)
    count = O.lb_stats(o_f["logits"], o_f["topk_idx"], cfg.E, G)["count"]
    print(f"[{name}] capacity {C}, dropped {int(o_f['dropped'].sum())} of {cfg.T * cfg.k}",
          flush=True)
    assert o_f["dropped"].sum() > 0

    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=G, gather=gather,
                     capacity_factor=factor, aux_coef=aux_coef, z_coef=z_coef)
    assert layer.capacity == C
    t = {key: dev(v, act) for key, v in inp.items() if key != "wr"}
    t["wr"] = dev(inp["wr"], torch.float32)
    layer.route(t["x"], t["wr"])
    # the oracle's routing and its block counts stand in for the router's
    layer.topk_idx.copy_(dev(o_f["topk_idx"], torch.int32))
    layer.topk_gate.copy_(dev(routing[1], torch.float32))
    layer.group_count.copy_(dev(count, torch.int32))
    layer.forward_experts(t["x"], t["w1"], t["w3"], t["w2"])
    layer.backward(t["dy"], t["x"], t["wr"], t["w1"], t["w3"], t["w2"])
    torch.cuda.synchronize()

    R = int(o_f["offsets"][-1])
    assert np.array_equal(host(layer.kept_idx), o_f["kept_idx"])
    assert np.array_equal(host(layer.group_dropped), o_f["dropped"])
    assert np.array_equal(host(layer.expert_offsets), o_f["offsets"])
    assert np.array_equal(host(layer.pos), o_f["pos"])
    assert np.array_equal(host(layer.src_token)[:R], o_f["src"][:R])
    if not gather:
        assert np.array_equal(host(layer.x_perm)[:R], inp["x"][o_f["src"][:R]])
    assert rel_err(host(layer.group_z), O.z_loss_groups(o_f["logits"], G)) <= TOL_ROUTER
    got, ex, bd = layer_floats(layer, o_f, o_b, B)
    check_floats(name, got, ex, bd, TOL[cfg.act], bound_only_keys(cfg))
    # dropped slots: no gradient through the combine
    assert np.all(host(layer.dgate)[o_f["kept_idx"] < 0] == 0.0)


def test_variants_on_an_empty_batch():
    """T = 0: nothing dropped, zero z-loss values, a zero router weight gradient."""
    _announce("variants T=0")
    E, k, d, G = 8, 2, 64, 2
    dims = M.make_dims(0, d, E, 64, k, torch.bfloat16)
    ws = M.alloc_workspace(dims, G)
    empty_i = torch.empty((1, k), dtype=torch.int32, device="cuda")[:0]
    dropped = torch.full((G,), -1, dtype=torch.int32, device="cuda")
    M.moe_capacity(dims, G, 4, empty_i, torch.empty_like(empty_i), dropped, ws)
    dwr = torch.full((E, d), float("nan"), device="cuda")
    e_f = torch.empty((1, k), device="cuda")[:0]
    M.moe_route_bwd_dense(dims, torch.empty((1, d), dtype=torch.bfloat16, device="cuda")[:0],
                          torch.zeros((E, d), device="cuda"),
                          torch.empty((1, E), device="cuda")[:0], empty_i, e_f, e_f, empty_i,
                          None, G, torch.zeros((G, E), dtype=torch.int32, device="cuda"), 0.01,
                          0.001, torch.empty((1, d), dtype=torch.bfloat16, device="cuda")[:0],
                          dwr, None, ws)
    torch.cuda.synchronize()
    assert np.all(host(dropped) == 0)
    assert np.all(host(dwr) == 0.0)
