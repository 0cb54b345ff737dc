"""GPU: expert-parallel dispatch emulated on one device.  The send buffer of
the deduplicated plan (one row per (group, token)) against the oracle's, and
its re-expansion into expert-contiguous rows against the permutation's x_perm,
bit for bit, at a small ragged size and at the C5 size (every row of the send
buffer against the oracle's) with both placements (contiguous and greedy
co-selection) for 8 and 16 groups.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import get_config, make_layer_inputs, stream
import top_routing_grouped_router_amd as M
from top_routing_grouped_router_amd import MoELayer

from _util import act_torch, dev, host

pytestmark = pytest.mark.gpu


def _plan(T, k, E, G, d_idx, pl):
    out = {n: torch.empty(s, dtype=torch.int32, device="cuda") for n, s in
           (("n_dest", T), ("group_rows", G), ("group_offsets", G + 1),
            ("row_token", max(T * k, 1)), ("assign_row", (T, k)), ("stats", 4))}
    ws = torch.empty(M.workspace_bytes(M.make_dims(T, 64, E, 64, k, 1), G), dtype=torch.uint8,
                     device="cuda")
    M.moe_dispatch_plan(T, k, E, G, d_idx, pl, out["n_dest"], out["group_rows"],
                        out["group_offsets"], out["row_token"], out["assign_row"], out["stats"],
                        ws)
    return out


def _check_case(T, d, E, k, act, x_np, idx_np, G, pl, oracle_send):
    ta = act_torch(act)
    layer = MoELayer(T, d, E, d, k, ta)
    dm = layer.dims
    x = dev(x_np, ta)
    d_idx = dev(idx_np, torch.int32)
    layer.topk_idx.copy_(d_idx)
    M.moe_permute(dm, layer.topk_idx, layer.expert_counts, layer.expert_offsets, layer.pos,
                  layer.src_token, x, layer.x_perm, layer.workspace)
    plan = _plan(T, k, E, G, d_idx, pl)
    send = torch.zeros(max(T * k, 1), d, dtype=ta, device="cuda")[:T * k]
    M.moe_dispatch_pack(dm, G, x, plan["group_offsets"], plan["row_token"], send)
    xp = torch.empty_like(layer.x_perm)
    M.moe_dispatch_expand(dm, send, plan["assign_row"], layer.pos, xp)
    torch.cuda.synchronize()
    assert torch.equal(xp, layer.x_perm), "expand(pack(x)) != x_perm"
    n = int(host(plan["group_offsets"])[G])
    if oracle_send is not None:
        o = O.dispatch_plan(idx_np, pl, G)
        ref = O.dispatch_pack(x_np, o["row_token"], o["rows_total"])
        assert n == o["rows_total"]
        assert np.array_equal(host(send)[:n], ref)
    # rows past the plan's total are not written
    assert not torch.any(send[n:] != 0)
    return n


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_ep_dispatch_small(act):
    print(f"\n[case] ep dispatch small {act}", flush=True)
    T, d, E, k, G = 200, 64, 16, 4, 4
    g = stream(60, 1)
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = g.standard_normal((T, d)).astype(np.float32)
    if act == "bf16":
        x = host(torch.from_numpy(x).to(torch.bfloat16))
    pl = np.array(stream(61, 1).permutation(np.arange(E) % G))
    _check_case(T, d, E, k, act, x, idx, G, pl, oracle_send=True)


def test_ep_dispatch_c5():
    print("\n[case] ep dispatch c5", flush=True)
    cfg = get_config("c5")
    inp = make_layer_inputs(cfg, parts=("x", "wr"))
    fit = make_layer_inputs(cfg, batch_seed=1, parts=("x",))
    idx = O.route(inp["x"], inp["wr"], cfg.k)["topk_idx"].astype(np.int32)
    idx_fit = O.route(fit["x"], inp["wr"], cfg.k)["topk_idx"]
    W_fit = O.coselect(idx_fit, cfg.E)
    for G in cfg.plan_groups:
        greedy = O.placement_greedy(W_fit, G)
        for kind, pl in (("contiguous", O.placement_contiguous(cfg.E, G)), ("correlated", greedy)):
            n = _check_case(cfg.T, cfg.d, cfg.E, cfg.k, cfg.act, inp["x"], idx, G, pl,
                            oracle_send=True)
            print(f"[c5 G={G} {kind}] rows {n} of {cfg.T * cfg.k}", flush=True)
