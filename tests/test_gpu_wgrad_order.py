"""GPU: the big-tile weight gradients (256 x 256 tiles, a reduction over each
expert's rows) on planted expert segments, against the exact fp64 oracle
(oracle.expert_weight_grads on the same bf16 operands), element by element.

The tiles of one product of one expert run together on one XCD, and the
groups are dealt by the experts' row counts, largest first (equal counts by
expert id).  The segments here reach what that order has to get right: experts
without rows (their gradient is zero), many experts with equal counts, a group
count (3 E) that leaves some XCDs without a group in the last round, ragged
counts that are not multiples of the 32-row step, and one expert far larger
than the rest.  Each case runs the materialised, the gathered (identity table)
and the gate-folded forms of the call; all three must agree bit for bit, and
every element must lie within twice its first-order bound: the bf16 rounding
of the result plus fp32 accumulation over the expert's rows,
|g - o| <= 2 (2^-8 |o| + gamma_K sum |terms|).
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import stream
import top_routing_grouped_router_amd._lib as L

pytestmark = pytest.mark.gpu

CASES = {
    # name: (d, f, rows per expert)
    "E13_empty_ties_ragged": (1024, 1024, [0, 700, 700, 2500, 64, 0, 31, 700, 1300, 5, 900,
                                           256, 1]),
    "E21_equal_counts": (1024, 1024, [256] * 9 + [0] + [256] * 9 + [0, 4000]),
}


def _bf16(rng, shape, scale=1.0):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(a).to("cuda", torch.bfloat16).contiguous()


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_big_tile_weight_gradients_on_planted_segments(name):
    print(f"\n[case] wgrad order {name}", flush=True)
    d, f, rows = CASES[name]
    E = len(rows)
    R = int(sum(rows))
    off_np = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    dm = L.make_dims(R, d, E, f, 1, torch.bfloat16)
    assert 3 * E * (d // 256) * (f // 256) >= 512, "the big-tile weight gradient needs the tiles"
    rng = stream(11, 500 + list(CASES).index(name))
    x = _bf16(rng, (R, d))
    dy = _bf16(rng, (R, d))
    h, da, db = (_bf16(rng, (R, f)) for _ in range(3))
    off = torch.from_numpy(off_np).cuda()
    src = torch.arange(R, dtype=torch.int32, device="cuda")
    ws = L.alloc_workspace(dm)

    outs = {}
    for form in ("materialised", "gathered", "folded"):
        dws = [torch.full((E, f, d), float("nan"), device="cuda", dtype=torch.bfloat16),
               torch.full((E, f, d), float("nan"), device="cuda", dtype=torch.bfloat16),
               torch.full((E, d, f), float("nan"), device="cuda", dtype=torch.bfloat16)]
        if form == "materialised":
            L.moe_expert_wgrad(dm, x, off, h, dy, da, db, *dws, ws)
        elif form == "gathered":
            L.moe_expert_wgrad_gather(dm, x, src, off, h, dy, da, db, *dws, ws)
        else:
            L.moe_expert_wgrad_folded(dm, x, dy, src, off, h, da, db, *dws)
        torch.cuda.synchronize()
        outs[form] = dws
    for form in ("gathered", "folded"):
        for u, v, key in zip(outs["materialised"], outs[form], ("dw1", "dw3", "dw2")):
            assert torch.equal(u, v), f"{form} {key}"

    xo, dyo, ho, dao, dbo = (_host(t) for t in (x, dy, h, da, db))
    ref = O.expert_weight_grads(xo, off_np, ho, dyo, dao, dbo, E)
    mag = O.expert_weight_grads(np.abs(xo), off_np, np.abs(ho), np.abs(dyo), np.abs(dao),
                                np.abs(dbo), E)
    for key, g in zip(("dw1", "dw3", "dw2"), outs["materialised"]):
        got = _host(g)
        o = ref[key]
        worst = 0.0
        for e in range(E):
            K = rows[e]
            if K == 0:
                assert not got[e].any(), f"{key} expert {e} without rows is not zero"
                continue
            bound = 2.0 * (O.U_BF16 * np.abs(o[e]) + O.gamma(K) * mag[key][e])
            diff = np.abs(got[e] - o[e])
            ratio = float((diff / np.maximum(bound, 1e-300)).max())
            worst = max(worst, ratio)
            assert np.all(diff <= bound), f"{key} expert {e} ({K} rows): {ratio:.2f} of the bound"
        print(f"[{name}] {key}: max |g - o| / bound = {worst:.3f}", flush=True)
