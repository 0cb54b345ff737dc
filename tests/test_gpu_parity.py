"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle,
on the materialised, unfolded path (x_perm written by moe_permute, the gate
applied in the combine, dy_perm from moe_combine_bwd); the default gathered,
gate-folded path is covered at every workload's full size in
test_gpu_default_path.py.

Rules (per output tensor):
  * integer and index outputs (routing outside near-ties, counts, offsets,
    permutation, dispatch plan, co-selection): bit-exact;
  * routing: identical expert sets wherever the oracle's top-k margin is at
    least 1e-3; where it is smaller (a near-tie) the GPU's set must still be a
    valid top-k of the oracle's logits to within fp32 resolution;
  * floats: every element within C_BOUND times its first-order error bound
    around the exact fp64 layer, and the row-normwise error within 1e-4
    (fp32 workloads and the router's fp32 outputs) or 2e-2 (bf16 workloads)
    outside the weight gradients of clustered-input workloads.
Downstream of the router, both sides run on the oracle's routing decision
(uploaded to the GPU), so float parity is judged on identical routing.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import get_config, make_layer_inputs, stream
from top_routing_grouped_router_amd import MoELayer
import top_routing_grouped_router_amd as M

from _parity import (bound_only_keys, check_plan, check_route, exact_reference, layer_floats,
                     oracle_routing)
from _util import TOL, act_torch, check_floats, dev, host

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"\n[case] {name}", flush=True)


# ---------------------------------------------------------------- whole layer

def run_layer(cfg, inp, G=1, backward=True, routing=None):
    """Forward (and backward) on the GPU with the given routing injected."""
    act = act_torch(cfg.act)
    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, n_groups=G)
    t = {k: dev(v, act) for k, v in inp.items() if k != "wr"}
    t["wr"] = dev(inp["wr"], torch.float32)
    layer.forward(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], routing=routing)
    if backward:
        layer.backward(t["dy"], t["x"], t["wr"], t["w1"], t["w3"], t["w2"])
    torch.cuda.synchronize()
    return layer


def compare_layer(label, cfg, inp, layer, routing, backward=True):
    """The layer's outputs against the exact oracle on the same routing."""
    o_f, o_b, B = exact_reference(inp, cfg.k, routing, backward=backward, act=cfg.act)
    check_plan(layer, o_f)
    R = int(o_f["offsets"][-1])
    # the permutation moves bits: x_perm[p] == x[src[p]] exactly
    assert np.array_equal(host(layer.x_perm)[:R], inp["x"][o_f["src"][:R]])
    got, ex, bd = layer_floats(layer, o_f, o_b, B)
    check_floats(label, got, ex, bd, TOL[cfg.act], bound_only_keys(cfg))
    return o_f, o_b


SMALL_CASES = {
    # name: (T, d, E, f, k, act)   -- several tiles, ragged rows and columns
    "ragged_bf16": (1000, 256, 8, 192, 3, "bf16"),
    "ragged_f32": (777, 128, 6, 128, 2, "f32"),
    "k_equals_E": (37, 64, 4, 64, 4, "bf16"),
    "single_expert_dense": (300, 64, 1, 64, 1, "f32"),
    "max_experts_max_k": (260, 64, 256, 64, 16, "bf16"),
    "wide_f_bf16": (513, 128, 5, 320, 2, "bf16"),
}


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_layer_small_cases(name):
    _announce(name)
    T, d, E, f, k, act = SMALL_CASES[name]
    cfg = get_config("c2", T=T, d=d, E=E, f=f, k=k, act=act, x_kind="normal", backward=True)
    inp = make_layer_inputs(cfg, seed=100 + list(SMALL_CASES).index(name))
    layer0 = MoELayer(T, d, E, f, k, act_torch(act))
    o_route, _ = check_route(layer0, inp["x"], inp["wr"], k)
    routing = (o_route["topk_idx"], o_route["gates"].astype(np.float32))
    layer = run_layer(cfg, inp, routing=oracle_routing(o_route))
    compare_layer(name, cfg, inp, layer, routing)
    if E == 1:
        assert np.all(host(layer.dwr) == 0.0)


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_layer_full_config(name):
    """Element-by-element parity at the workload's full size (C1's backward
    too: the fp32 backward kernels at that size)."""
    _announce(name)
    cfg = get_config(name)
    inp = make_layer_inputs(cfg, with_dy=True)
    G = max(cfg.lb_groups)
    layer0 = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act_torch(cfg.act), n_groups=G)
    o_route, _ = check_route(layer0, inp["x"], inp["wr"], cfg.k, G=G)
    routing = (o_route["topk_idx"], o_route["gates"].astype(np.float32))
    layer = run_layer(cfg, inp, G=G, routing=oracle_routing(o_route))
    compare_layer(name, cfg, inp, layer, routing)


# ---------------------------------------------------------------- invariants

def test_route_exact_ties_pick_lower_id():
    _announce("exact ties")
    T, d, E, k = 256, 64, 8, 3
    g = stream(31, 1)
    wr = g.standard_normal((E, d)).astype(np.float32)
    wr[5] = wr[2]          # experts 2 and 5 always tie exactly
    wr[7] = wr[0]
    x = g.standard_normal((T, d)).astype(np.float32)
    layer = MoELayer(T, d, E, 64, k, torch.float32)
    o, same = check_route(layer, x, wr, k)
    idx = host(layer.topk_idx)
    assert np.array_equal(idx, o["topk_idx"])
    for t in range(T):
        row = list(idx[t])
        if 5 in row:
            assert 2 in row and row.index(2) < row.index(5)


def test_bitwise_rerun_and_layout_invariance():
    """Two runs give identical bytes; the LB-statistics grouping does not
    change any layer output (only the per-group statistics)."""
    _announce("determinism")
    cfg = get_config("c2", T=4096)
    inp = make_layer_inputs(cfg)
    outs = []
    for G in (1, 1, 8):
        layer = run_layer(cfg, inp, G=G)
        outs.append({k: host(getattr(layer, k)).copy() for k in
                     ("logits", "topk_idx", "topk_gate", "y", "dx", "dw1", "dw3", "dw2", "dwr",
                      "dgate")})
    for k in outs[0]:
        assert np.array_equal(outs[0][k].view(np.uint8), outs[1][k].view(np.uint8)), k
        assert np.array_equal(outs[0][k].view(np.uint8), outs[2][k].view(np.uint8)), k


def test_kernel_phases_match_coarse_calls():
    """moe_expert_* phases give the same bytes as moe_grouped_swiglu_fwd/bwd."""
    _announce("phases")
    for name in ("c2", "c3"):
        cfg = get_config(name, T=2048)
        inp = make_layer_inputs(cfg)
        layer = run_layer(cfg, inp)
        dm, act = layer.dims, act_torch(cfg.act)
        w1, w3, w2 = (dev(inp[k], act) for k in ("w1", "w3", "w2"))
        a, b, h = (torch.empty_like(layer.a) for _ in range(3))
        y = torch.empty_like(layer.y_perm)
        M.moe_expert_up(dm, layer.x_perm, layer.expert_offsets, w1, w3, a, b, h)
        M.moe_expert_down(dm, h, layer.expert_offsets, w2, y)
        da, db = torch.empty_like(layer.a), torch.empty_like(layer.a)
        dxp = torch.empty_like(layer.dx_perm)
        dw1, dw3, dw2 = (torch.empty_like(t) for t in (layer.dw1, layer.dw3, layer.dw2))
        M.moe_expert_dgrad_down(dm, layer.dy_perm, layer.expert_offsets, w2, a, b, da, db)
        M.moe_expert_dgrad_up(dm, da, db, layer.expert_offsets, w1, w3, dxp)
        M.moe_expert_wgrad(dm, layer.x_perm, layer.expert_offsets, h, layer.dy_perm, da, db,
                           dw1, dw3, dw2, layer.workspace)
        torch.cuda.synchronize()
        for got, ref in ((a, layer.a), (b, layer.b), (h, layer.h), (y, layer.y_perm),
                         (dxp, layer.dx_perm), (dw1, layer.dw1), (dw3, layer.dw3),
                         (dw2, layer.dw2)):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_empty_batch():
    _announce("T=0")
    cfg = get_config("c2", T=0, d=64, E=4, f=64, k=2)
    layer = MoELayer(0, 64, 4, 64, 2, torch.bfloat16)
    z = torch.zeros(1, 64, dtype=torch.bfloat16, device="cuda")[:0]
    w = torch.ones(4, 64, 64, dtype=torch.bfloat16, device="cuda")
    wr = torch.ones(4, 64, dtype=torch.float32, device="cuda")
    layer.dw1.fill_(7)
    layer.dwr.fill_(7)
    layer.step(z, wr, w, w, w, z)
    torch.cuda.synchronize()
    assert int(host(layer.near_tie_count)[0]) == 0
    assert np.all(host(layer.expert_counts) == 0) and np.all(host(layer.expert_offsets) == 0)
    assert np.all(host(layer.dw1) == 0) and np.all(host(layer.dwr) == 0)
    assert np.all(host(layer.group_count) == 0)


# ---------------------------------------------------------------- index products

@pytest.mark.parametrize("name", ["c4", "c5"])
def test_dispatch_plan_and_coselect(name):
    _announce(f"plan {name}")
    cfg = get_config(name)
    inp = make_layer_inputs(cfg, parts=("x", "wr"))
    fit = make_layer_inputs(cfg, batch_seed=1, parts=("x",))
    idx = O.route(inp["x"], inp["wr"], cfg.k)["topk_idx"]
    idx_fit = O.route(fit["x"], inp["wr"], cfg.k)["topk_idx"]
    d_idx = dev(idx, torch.int32)
    W = torch.empty(cfg.E, cfg.E, dtype=torch.int32, device="cuda")
    M.moe_coselect(cfg.T, cfg.k, cfg.E, d_idx, W)
    torch.cuda.synchronize()
    W_o = O.coselect(idx, cfg.E)
    assert np.array_equal(host(W), W_o)
    W_fit = O.coselect(idx_fit, cfg.E)
    for G in cfg.plan_groups:
        greedy = M.moe_placement_greedy(cfg.E, G, W_fit)
        assert greedy == [int(v) for v in O.placement_greedy(W_fit, G)]
        for kind, pl in (("contiguous", O.placement_contiguous(cfg.E, G)), ("correlated", greedy)):
            T, k = cfg.T, cfg.k
            out = {n: torch.empty(s, dtype=torch.int32, device="cuda") for n, s in
                   (("n_dest", T), ("group_rows", G), ("group_offsets", G + 1),
                    ("row_token", T * k), ("assign_row", (T, k)), ("stats", 4))}
            ws = torch.empty(M.workspace_bytes(M.make_dims(T, 64, cfg.E, 64, k, 1), G),
                             dtype=torch.uint8, device="cuda")
            M.moe_dispatch_plan(T, k, cfg.E, G, d_idx, pl, out["n_dest"], out["group_rows"],
                                out["group_offsets"], out["row_token"], out["assign_row"],
                                out["stats"], ws)
            torch.cuda.synchronize()
            o = O.dispatch_plan(idx, pl, G)
            R = o["rows_total"]
            assert np.array_equal(host(out["n_dest"]), o["n_dest"])
            assert np.array_equal(host(out["group_rows"]), o["group_rows"])
            assert np.array_equal(host(out["group_offsets"]), o["group_offsets"])
            assert np.array_equal(host(out["row_token"])[:R], o["row_token"])
            assert np.array_equal(host(out["assign_row"]), o["assign_row"])
            assert list(host(out["stats"])) == [R, o["rows_removed"], o["tokens_single_group"],
                                                o["rows_off_home"]]
            print(f"[{name} G={G} {kind}] same-group {o['same_group_share']:.3f} "
                  f"destinations {o['mean_destinations']:.3f} dedup {o['dedup_fraction']:.3f}",
                  flush=True)


# ---------------------------------------------------------------- permutation edge cases

@pytest.mark.parametrize("T,E,k,rep", [(2048, 8, 4, False), (2048, 8, 4, True), (2049, 8, 4, False),
                                         (16384, 64, 6, False), (16384, 64, 6, True),
                                         (32768, 64, 2, False), (40000, 16, 4, False)])
def test_plan_with_gates_follows_the_definition(T, E, k, rep):
    """moe_permute_gates (the plan alone, with the gates carried into row
    order) on each of its kernel forms, bit for bit against the oracle's plan:
    up to 8192 assignments one kernel counts the ids itself (T = 2048, k = 4),
    above it a histogram kernel comes first (T = 2049), up to 128 blocks of 256
    tokens the scan and scatter are one kernel (T = 16384, 32768), beyond
    that they are separate (T = 40000).  rep: some tokens repeat an expert
    (outside the routing contract; every slot still gets its own row)."""
    _announce(f"plan with gates T={T} E={E} k={k} repeats={rep}")
    from synth import make_routing
    idx = make_routing(T, E, k, seed=T + k).astype(np.int32)
    g = stream(78, T)
    if rep:
        rows = g.choice(T, size=max(3, T // 50), replace=False)
        idx[rows, 1] = idx[rows, 0]
    gate = g.random((T, k)).astype(np.float32)
    plan = O.permute_plan(idx, E)
    R = T * k
    dims = M.make_dims(T, 64, E, 64, k, torch.bfloat16)
    ws = M.alloc_workspace(dims, 1)
    out = {n: torch.full(sh, -7, dtype=torch.int32, device="cuda") for n, sh in
           (("counts", (E,)), ("offsets", (E + 1,)), ("pos", (T, k)), ("src", (R,)))}
    gp = torch.full((R,), -1.0, device="cuda")
    M.moe_permute_gates(dims, dev(idx, torch.int32), dev(gate, torch.float32), out["counts"],
                        out["offsets"], out["pos"], out["src"], gp, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["counts"]), plan["counts"])
    assert np.array_equal(host(out["offsets"]), plan["offsets"])
    assert np.array_equal(host(out["pos"]), plan["pos"])
    assert np.array_equal(host(out["src"]), plan["src"])
    want = np.zeros(R, np.float32)
    want[plan["pos"].reshape(-1)] = gate.reshape(-1)
    assert np.array_equal(host(gp), want)


@pytest.mark.parametrize("T,E,k", [(1000, 8, 3), (40000, 16, 4)])
def test_permute_follows_the_definition_with_repeated_ids(T, E, k):
    """A token that lists an expert twice is outside the routing contract, but
    the sort is still the definition's: every slot gets its own row, in slot
    order, with x_perm[pos] = x bit for bit.  T = 1000 takes the fused
    scan/scatter/gather kernel, T = 40000 (157 blocks) the separate kernels;
    a clean table of the larger size is checked too."""
    _announce(f"permute repeated ids T={T} E={E} k={k}")
    from synth import make_routing
    d = 64
    idx = make_routing(T, E, k, seed=T).astype(np.int32)
    clean = idx.copy()
    g = stream(77, T)
    rows = g.choice(T, size=max(3, T // 50), replace=False)
    idx[rows, 1] = idx[rows, 0]                 # slot 1 repeats slot 0
    x = g.standard_normal((T, d)).astype(np.float32)
    for table in (idx, clean):
        plan = O.permute_plan(table, E)
        dims = M.make_dims(T, d, E, 64, k, torch.float32)
        ws = M.alloc_workspace(dims, 1)
        out = {n: torch.full(s, -7, dtype=torch.int32, device="cuda") for n, s in
               (("counts", (E,)), ("offsets", (E + 1,)), ("pos", (T, k)), ("src", (T * k,)))}
        xp = torch.zeros(T * k, d, device="cuda")
        M.moe_permute(dims, dev(table, torch.int32), out["counts"], out["offsets"], out["pos"],
                      out["src"], dev(x, torch.float32), xp, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(out["counts"]), plan["counts"])
        assert np.array_equal(host(out["offsets"]), plan["offsets"])
        assert np.array_equal(host(out["pos"]), plan["pos"])
        assert np.array_equal(host(out["src"]), plan["src"])
        assert np.array_equal(host(xp), x[plan["src"]])
