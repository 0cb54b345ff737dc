"""GPU checks of the routing-fragility probe: moe_route_flips against the
oracle's set comparison (bit-exact), and the probe itself -- moving one
router weight by m units in the last place flips a token's expert set only
where that weight's logit shift reaches the token's routing margin."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import get_config, make_layer_inputs, make_routing, stream
import top_routing_grouped_router_amd as M

from _util import dev, host

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"\n[case] {name}", flush=True)


@pytest.mark.parametrize("T,E,k", [(1000, 8, 2), (4096, 256, 16), (333, 64, 6)])
def test_route_flips_bit_exact(T, E, k):
    _announce(f"route_flips T={T} E={E} k={k}")
    a = make_routing(T, E, k, seed=1)
    b = a.copy()
    g = stream(92, T)
    rows = g.permutation(T)
    for t in rows[: T // 3]:             # same set, other slot order: no flip
        b[t] = b[t][g.permutation(k)]
    for t in rows[T // 3: T // 2]:       # one expert replaced: a flip
        free = np.setdiff1d(np.arange(E), b[t])
        b[t, g.integers(0, k)] = g.choice(free)
    flips = torch.full((T,), -1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    M.moe_route_flips(T, k, E, dev(a, torch.int32), dev(b, torch.int32), flips, n)
    torch.cuda.synchronize()
    ref = O.route_flips(a, b)
    assert np.array_equal(host(flips).astype(bool), ref)
    assert int(host(n)[0]) == int(ref.sum()) == T // 2 - T // 3


@pytest.mark.parametrize("m", [1, 1 << 20])
def test_one_weight_nudge_flips_only_within_its_logit_shift(m):
    _announce(f"nudge {m} ulp")
    cfg = get_config("c2")
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    inp = make_layer_inputs(cfg, parts=("x", "wr"))
    x, wr = inp["x"], inp["wr"]
    e, i = 3, int(np.argmax(np.abs(wr[3])))
    wn = O.nudge_ulps(wr, e, i, m)
    dims = M.make_dims(T, d, E, cfg.f, k, torch.bfloat16)
    ws = M.alloc_workspace(dims, 1)
    xd = dev(x, torch.bfloat16)
    out = []
    for w in (wr, wn):
        lg = torch.empty((T, E), device="cuda")
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        gate = torch.empty((T, k), device="cuda")
        mg = torch.empty(T, device="cuda")
        ntc = torch.empty(1, dtype=torch.int32, device="cuda")
        M.moe_route(dims, xd, dev(w, torch.float32), lg, idx, gate, mg, 1e-3, ntc, 1, None, None,
                    None, ws)
        out.append((idx, mg, lg))
    flips = torch.empty(T, dtype=torch.int32, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    M.moe_route_flips(T, k, E, out[0][0], out[1][0], flips, n)
    torch.cuda.synchronize()
    fl = host(flips).astype(bool)
    assert np.array_equal(fl, O.route_flips(host(out[0][0]), host(out[1][0])))
    shift = np.abs(x[:, i].astype(np.float64) * (float(wn[e, i]) - float(wr[e, i])))
    lg = host(out[0][2]).astype(np.float64)
    slack = 1e-5 * float(np.sqrt(np.mean(lg ** 2)))       # fp32 rounding of the logits
    margin = host(out[0][1]).astype(np.float64)
    print(f"[nudge {m}] flips {int(fl.sum())} of {T}; largest shift {shift.max():.2e}", flush=True)
    assert np.all(margin[fl] <= shift[fl] + slack)
    # the oracle's prediction from exact logits agrees wherever it is clear
    la = O.router_logits(x, wr)
    lb = O.router_logits(x, wn)
    others = np.sort(np.delete(la, e, axis=1), axis=1)[:, ::-1][:, k - 1]
    inside = (O.topk_select(la, k)[0] == e).any(axis=1)
    pred = np.where(inside, lb[:, e] < others, lb[:, e] > others)
    clear = (np.abs(lb[:, e] - others) > 4 * slack) & (np.abs(la[:, e] - others) > 4 * slack)
    assert np.array_equal(fl[clear], pred[clear])
    if m > 1:
        assert fl.sum() > 0
