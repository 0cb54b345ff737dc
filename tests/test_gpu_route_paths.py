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
