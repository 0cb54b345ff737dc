"""GPU: the router for long rows (bf16 hidden states, E <= 64, d > 256: the
streaming router, fp32 Wr split in registers) and the kernel that folds its
per-tile partials per balancing block, held to the routing rules of
check_route (logits, expert sets, gates, margins, near-ties and the per-block
balancing statistics against the fp64 oracle).

The cases cover widths from 512 to 4096, expert
counts that fill 1, 2 and 4 16-expert tiles (and pad 3 to 4), 1 to 64
balancing blocks (the fold runs one workgroup per block) and token counts
with a ragged last tile.
"""
import pytest

from synth import get_config, make_layer_inputs
from top_routing_grouped_router_amd import MoELayer

from _parity import check_route
from _util import act_torch

pytestmark = pytest.mark.gpu

CASES = {
    # name: (T, d, E, k, G)
    "d512_E4": (4096, 512, 4, 2, 1),
    "d512_E8_G2": (4096, 512, 8, 2, 2),
    "d768_E64_G8": (2048, 768, 64, 2, 8),
    "d1024_E20_G3": (6144, 1024, 20, 3, 3),
    "d1536_E40_G4": (8192, 1536, 40, 4, 4),
    "d2048_E64_ragged_T": (3000, 2048, 64, 6, 1),
    "d2560_E16_ragged_T": (1000, 2560, 16, 4, 1),
    "d3584_E33_G2": (512, 3584, 33, 5, 2),
    "d4096_E64_64_blocks": (16384, 4096, 64, 8, 64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_route_paths(name):
    T, d, E, k, G = CASES[name]
    print(f"\n[case] route {name} T={T} d={d} E={E} k={k} G={G}", flush=True)
    cfg = get_config("c2", T=T, d=d, E=E, f=64, k=k, act="bf16", x_kind="normal",
                     backward=False)
    inp = make_layer_inputs(cfg, seed=400 + list(CASES).index(name), parts=("x", "wr"))
    layer = MoELayer(T, d, E, 64, k, act_torch("bf16"), n_groups=G)
    check_route(layer, inp["x"], inp["wr"], k, G=G)


BWD_CASES = {
    # name: (T, d, E, k)   -- bf16 X, d >= 1024: the router weight gradient on
    # the matrix cores (16, 32 and 64 expert rows; k compiled and runtime)
    "d1024_E5_k1": (777, 1024, 5, 1),
    "d1024_E20_k3_ragged_T": (1000, 1024, 20, 3),
    "d2048_E33_k8": (2048, 2048, 33, 8),
    "d1280_E64_k10": (1500, 1280, 64, 10),
    "d1024_E8_one_token": (1, 1024, 8, 2),
    "d2048_E64_31_tokens": (31, 2048, 64, 6),
}


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_router_backward_wide_rows(name):
    """dWr and dX of a layer step on the oracle's routing, against the exact
    fp64 oracle within the first-order error bounds and the bf16 tolerance."""
    from _parity import exact_reference, layer_floats, oracle_routing
    from _util import TOL, check_floats, dev
    import numpy as np
    import torch

    T, d, E, k = BWD_CASES[name]
    print(f"\n[case] router backward {name}", flush=True)
    cfg = get_config("c2", T=T, d=d, E=E, f=64, k=k, act="bf16", x_kind="normal",
                     backward=True)
    inp = make_layer_inputs(cfg, seed=500 + list(BWD_CASES).index(name))
    probe = MoELayer(T, d, E, 64, k, torch.bfloat16)
    o_route, _ = check_route(probe, inp["x"], inp["wr"], k)
    routing = (o_route["topk_idx"], o_route["gates"].astype(np.float32))
    layer = MoELayer(T, d, E, 64, k, torch.bfloat16)
    t = {key: dev(v, torch.bfloat16) for key, v in inp.items() if key != "wr"}
    t["wr"] = dev(inp["wr"], torch.float32)
    layer.forward(t["x"], t["wr"], t["w1"], t["w3"], t["w2"], routing=oracle_routing(o_route))
    layer.backward(t["dy"], t["x"], t["wr"], t["w1"], t["w3"], t["w2"])
    torch.cuda.synchronize()
    o_f, o_b, B = exact_reference(inp, k, routing, act="bf16")
    got, ex, bd = layer_floats(layer, o_f, o_b, B)
    keys = ("dwr", "dx")
    # with only a few tokens per expert (T k < 64 E) each dWr row sums a few
    # terms of random sign, and the bf16 rounding upstream of dl (dgate from
    # bf16 rows) moves it by about 2e-2 of the row: held to the bound alone
    bound_only = ("dwr",) if T * k < 64 * E else ()
    check_floats(f"route bwd {name}", {q: got[q] for q in keys}, {q: ex[q] for q in keys},
                 {q: bd[q] for q in keys}, TOL["bf16"], bound_only)
