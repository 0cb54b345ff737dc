"""A whole layer step captured in a HIP graph: every replay, with eager work
and synchronisations in between and the outputs cleared before it, must give
the eager step's results bit for bit (the library launches on the caller's
stream and allocates, frees and synchronises nothing)."""
import numpy as np
import pytest
import torch

from synth import get_config, make_layer_inputs
from top_routing_grouped_router_amd import MoELayer

from _util import act_torch, dev, host

pytestmark = pytest.mark.gpu

OUTPUTS = ("logits", "topk_idx", "topk_gate", "margin", "near_tie_count", "group_count",
           "group_mean_prob", "group_aux", "expert_counts", "expert_offsets", "pos", "src_token",
           "y_perm", "y", "dgate", "dx_perm", "dw1", "dw3", "dw2", "dx", "dwr", "kept_idx",
           "group_dropped", "group_z", "dlogits", "gate_perm", "dgate_part", "da", "db")


@pytest.mark.parametrize("variant", ["default", "capacity_losses", "gate_folded"])
def test_layer_step_graph_replays_match_eager(variant):
    print(f"\n[case] graph {variant}", flush=True)
    cfg = get_config("c2", T=2048)
    inp = make_layer_inputs(cfg, seed=5, with_dy=True)
    act = act_torch(cfg.act)
    kw = dict(n_groups=4, gather=True)
    if variant == "capacity_losses":
        kw.update(capacity_factor=1.0, aux_coef=0.01, z_coef=0.001)
    if variant == "gate_folded":
        kw.update(fold_gate=True)
    layer = MoELayer(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act, **kw)
    t = {key: dev(v, act) for key, v in inp.items() if key != "wr"}
    t["wr"] = dev(inp["wr"], torch.float32)

    def step():
        layer.step(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], t["dy"])

    step()
    torch.cuda.synchronize()
    names = [n for n in OUTPUTS if getattr(layer, n) is not None]
    # permuted-row buffers are defined only for the offsets[E] kept rows
    kept = int(host(layer.expert_offsets)[-1])
    if variant == "capacity_losses":
        assert kept < cfg.T * cfg.k == kept + int(host(layer.group_dropped).sum())
    rows = {"src_token", "y_perm", "dx_perm", "gate_perm", "dgate_part", "da", "db"}

    def defined(name):
        a = host(getattr(layer, name))
        return a[:kept] if name in rows else a

    ref = {name: defined(name).copy() for name in names}

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device="cuda")
    for replay in range(4):
        for name in names:                       # clear every output before the replay
            buf = getattr(layer, name)
            buf.fill_(-7 if buf.dtype == torch.int32 else float("nan"))
        scratch.uniform_()                       # unrelated eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in names:
            got = defined(name)
            assert np.array_equal(got, ref[name], equal_nan=False), (variant, replay, name)
