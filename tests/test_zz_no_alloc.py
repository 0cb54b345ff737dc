"""GPU: the allocation-free router (moe_route_noalloc, scratch in a static
device array) against moe_route with a caller workspace.  The two run the
same kernels, so every output must agree bit for bit.  Two calls in a row on
the shared static scratch, the second with a smaller input (a different
kernel path: the streaming router at d = 2048, then the LDS router at d = 256
with 4 balancing blocks), then the first again."""
import numpy as np
import pytest
import torch

from synth import get_config, make_layer_inputs
import top_routing_grouped_router_amd._lib as L

from _util import act_torch, dev

pytestmark = pytest.mark.gpu

OUTS = ("logits", "idx", "gate", "margin", "ntc", "count", "P", "aux")


def _buffers(cfg, G):
    T, E, k = cfg.T, cfg.E, cfg.k
    f32 = dict(dtype=torch.float32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    return {"logits": torch.full((T, E), float("nan"), **f32), "idx": torch.full((T, k), -7, **i32),
            "gate": torch.full((T, k), float("nan"), **f32),
            "margin": torch.full((T,), float("nan"), **f32), "ntc": torch.full((1,), -7, **i32),
            "count": torch.full((G, E), -7, **i32), "P": torch.full((G, E), float("nan"), **f32),
            "aux": torch.full((G,), float("nan"), **f32)}


def _route(cfg, inp, G, noalloc):
    act = act_torch(cfg.act)
    dm = L.make_dims(cfg.T, cfg.d, cfg.E, cfg.f, cfg.k, act)
    x, wr = dev(inp["x"], act), dev(inp["wr"], torch.float32)
    o = _buffers(cfg, G)
    args = (dm, x, wr, o["logits"], o["idx"], o["gate"], o["margin"], 1e-3, o["ntc"], G,
            o["count"], o["P"], o["aux"])
    if noalloc:
        L.moe_route_noalloc(*args)
    else:
        L.moe_route(*args, L.alloc_workspace(dm, G))
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in o.items()}


def test_route_noalloc_matches_route_with_workspace():
    cases = [(get_config("c5"), 1), (get_config("c2", T=4096), 4), (get_config("c5"), 1)]
    for cfg, G in cases:
        print(f"\n[case] noalloc {cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} G={G}", flush=True)
        inp = make_layer_inputs(cfg, parts=("x", "wr"))
        ref = _route(cfg, inp, G, noalloc=False)
        got = _route(cfg, inp, G, noalloc=True)
        for n in OUTS:
            assert np.array_equal(got[n].view(np.uint8), ref[n].view(np.uint8)), (cfg.name, n)
        assert int(ref["ntc"][0]) >= 0 and np.isfinite(ref["P"]).all()
