"""Checks of the seeded input recipes (shapes, determinism, bf16 rounding and
the calibration of the correlated 64-centroid mixture)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import CONFIGS, bf16_bits, bf16_from_bits, bf16_round, get_config, make_layer_inputs, stream


def test_bf16_rounding_agrees_with_torch():
    g = stream(1, 1)
    a = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0, 65504.0], np.float32)])
    ours = bf16_round(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(bf16_from_bits(bf16_bits(a)), ours)


def test_streams_are_independent_of_draw_order():
    cfg = get_config("c2", T=256)
    full = make_layer_inputs(cfg)
    only_x = make_layer_inputs(cfg, parts=("x",))
    assert np.array_equal(full["x"], only_x["x"])
    again = make_layer_inputs(cfg)
    for key in full:
        assert np.array_equal(full[key], again[key])
    other = make_layer_inputs(cfg, batch_seed=1)
    assert not np.array_equal(full["x"], other["x"])
    assert np.array_equal(full["w1"], other["w1"])


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_shapes_and_dtypes(name):
    cfg = CONFIGS[name]
    inp = make_layer_inputs(cfg)
    assert inp["x"].shape == (cfg.T, cfg.d)
    assert inp["wr"].shape == (cfg.E, cfg.d)
    assert inp["w1"].shape == (cfg.E, cfg.f, cfg.d)
    assert inp["w2"].shape == (cfg.E, cfg.d, cfg.f)
    assert ("dy" in inp) == cfg.backward
    if cfg.act == "bf16":
        for key in ("x", "w1", "w3", "w2"):
            assert np.array_equal(bf16_round(inp[key]), inp[key])
    assert np.std(inp["wr"]) == pytest.approx(1 / np.sqrt(cfg.d), rel=0.05)


def test_mixture64_top20_pairs_carry_about_40pct_of_tokens():
    """The correlated mixture is calibrated so that about 1% of the expert pairs
    (20 of C(64,2)) carry about 40% of the tokens' top-2 selections."""
    cfg = CONFIGS["c4"]
    inp = make_layer_inputs(cfg, parts=("x", "wr"))
    r = O.route(inp["x"], inp["wr"], 2)
    W = O.coselect(r["topk_idx"], cfg.E)
    pair_counts = np.sort(W[np.triu_indices(cfg.E, 1)])[::-1]
    share = pair_counts[:20].sum() / cfg.T
    assert 0.37 <= share <= 0.43, share


def test_mixture32_gives_high_near_tie_rate():
    cfg = CONFIGS["c3"]
    inp = make_layer_inputs(cfg, parts=("x", "wr"))
    r = O.route(inp["x"], inp["wr"], cfg.k)
    assert r["near_tie"].mean() > 0.05
