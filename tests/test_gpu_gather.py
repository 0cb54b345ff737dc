"""GPU: the gathered-input calls (expert input row p read as X[src_token[p]])
against the calls on the materialised x_perm.  Both run the same arithmetic in
the same order on the same values, so the outputs must agree bit for bit.

Shapes are chosen to reach every kernel path the gathered calls have: the
persistent small tile (UP), the LDS-DMA big tile (UP; T=8192 d=f=1024 E=16
k=2), the small-tile weight-gradient ring with 8 stages (C2's grid) and with 4
(C3's), the split-K weight-gradient stream (few tiles), the big-tile
weight-gradient ring, and the fp32 path.
"""
import numpy as np
import pytest
import torch

from synth import stream
import top_routing_grouped_router_amd._lib as L
from top_routing_grouped_router_amd import MoELayer

from _util import act_torch

pytestmark = pytest.mark.gpu

CASES = {
    # name: (T, d, E, f, k, act)
    "small_split_k_bf16": (1000, 256, 8, 192, 3, "bf16"),
    "small_f32": (777, 128, 6, 128, 2, "f32"),
    "many_experts_bf16": (260, 64, 256, 64, 16, "bf16"),
    "c2_shape": (16384, 256, 16, 256, 4, "bf16"),
    "c3_shape": (16384, 256, 64, 64, 4, "bf16"),
    "big_tile": (8192, 1024, 16, 1024, 2, "bf16"),
}


def _rand(rng, shape, act, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(a).to("cuda", act_torch(act)).contiguous()


@pytest.mark.parametrize("name", list(CASES))
def test_gathered_calls_match_materialised(name):
    print(f"\n[case] gather {name}", flush=True)
    T, d, E, f, k, act = CASES[name]
    rng = stream(7, 100 + list(CASES).index(name))
    ta = act_torch(act)
    layer = MoELayer(T, d, E, f, k, ta)
    dm = layer.dims
    x = _rand(rng, (T, d), act)
    wr = _rand(rng, (E, d), "f32", d ** -0.5).float()
    w1, w3 = _rand(rng, (E, f, d), act, d ** -0.5), _rand(rng, (E, f, d), act, d ** -0.5)
    w2 = _rand(rng, (E, d, f), act, f ** -0.5)
    layer.route(x, wr)
    L.moe_permute(dm, layer.topk_idx, layer.expert_counts, layer.expert_offsets, layer.pos,
                  layer.src_token, x, layer.x_perm, layer.workspace)
    R = T * k
    off, src = layer.expert_offsets, layer.src_token

    # expert up: a, b, h
    outs = [[torch.empty(R, f, device="cuda", dtype=ta) for _ in range(3)] for _ in range(2)]
    L.moe_expert_up(dm, layer.x_perm, off, w1, w3, *outs[0])
    L.moe_expert_up_gather(dm, x, src, off, w1, w3, *outs[1])
    torch.cuda.synchronize()
    for u, v, key in zip(outs[0], outs[1], "abh"):
        assert torch.equal(u, v), f"up {key}"

    # weight gradients on arbitrary operands
    h, da, db = (_rand(rng, (R, f), act) for _ in range(3))
    dy = _rand(rng, (R, d), act)
    dws = [[torch.empty(E, f, d, device="cuda", dtype=ta), torch.empty(E, f, d, device="cuda",
            dtype=ta), torch.empty(E, d, f, device="cuda", dtype=ta)] for _ in range(2)]
    L.moe_expert_wgrad(dm, layer.x_perm, off, h, dy, da, db, *dws[0], layer.workspace)
    L.moe_expert_wgrad_gather(dm, x, src, off, h, dy, da, db, *dws[1], layer.workspace)
    torch.cuda.synchronize()
    for u, v, key in zip(dws[0], dws[1], ("dw1", "dw3", "dw2")):
        assert torch.equal(u, v), f"wgrad {key}"

    # the layer-level pair
    y = [torch.empty(R, d, device="cuda", dtype=ta) for _ in range(2)]
    abh = [[torch.empty(R, f, device="cuda", dtype=ta) for _ in range(3)] for _ in range(2)]
    L.moe_grouped_swiglu_fwd(dm, layer.x_perm, off, w1, w3, w2, *abh[0], y[0])
    L.moe_grouped_swiglu_fwd_gather(dm, x, src, off, w1, w3, w2, *abh[1], y[1])
    dx = [torch.empty(R, d, device="cuda", dtype=ta) for _ in range(2)]
    L.moe_grouped_swiglu_bwd(dm, layer.x_perm, off, w1, w3, w2, *abh[0], dy, dx[0], *dws[0],
                             layer.workspace)
    L.moe_grouped_swiglu_bwd_gather(dm, x, src, off, w1, w3, w2, *abh[0], dy, dx[1], *dws[1],
                                    layer.workspace)
    torch.cuda.synchronize()
    assert torch.equal(y[0], y[1]), "fwd y_perm"
    assert torch.equal(dx[0], dx[1]), "bwd dx_perm"
    for u, v, key in zip(dws[0], dws[1], ("dw1", "dw3", "dw2")):
        assert torch.equal(u, v), f"bwd {key}"


def test_gathered_layer_step_matches():
    """A whole layer step with the plan-only permutation and the gathered
    calls gives the same outputs as the materialised sequence."""
    print("\n[case] gather layer step", flush=True)
    T, d, E, f, k = 4096, 256, 16, 256, 4
    rng = stream(8, 1)
    x = _rand(rng, (T, d), "bf16")
    wr = _rand(rng, (E, d), "f32", d ** -0.5).float()
    w1, w3 = _rand(rng, (E, f, d), "bf16", d ** -0.5), _rand(rng, (E, f, d), "bf16", d ** -0.5)
    w2 = _rand(rng, (E, d, f), "bf16", f ** -0.5)
    dy = _rand(rng, (T, d), "bf16")
    ref = MoELayer(T, d, E, f, k, torch.bfloat16)
    ref.step(x, wr, w1, w3, w2, dy)
    gat = MoELayer(T, d, E, f, k, torch.bfloat16, gather=True)
    gat.step(x, wr, w1, w3, w2, dy)
    torch.cuda.synchronize()
    for key in ("y", "dx", "dw1", "dw3", "dw2", "dwr"):
        assert torch.equal(getattr(ref, key), getattr(gat, key)), key
