"""Seeded generators for the MoE-layer inputs.

Every tensor has its own random stream, PCG64 seeded with (seed, stream id), so
a tensor's values do not depend on which other tensors were drawn or in what
order.  Model tensors (router and expert weights, mixture centres) use the
model seed; token tensors (hidden states, mixture labels, upstream gradient)
use the batch seed.

bf16 workloads store X, W1, W3, W2 and dY in bfloat16: the fp32 draws are
rounded to nearest-even once, here, so that the GPU path and the oracle start
from the very same values.  The router weight stays fp32.
"""
from __future__ import annotations

import numpy as np

from .configs import Config

# stream ids
_S_WR, _S_W1, _S_W3, _S_W2 = 1, 2, 3, 4
_S_CENTRES = 5
_S_X, _S_DY, _S_LABELS, _S_NOISE = 10, 11, 12, 13
_S_ROUTE = 20


def stream(seed: int, stream_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream_id)])))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exactly equal fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 and return them as fp32."""
    return bf16_from_bits(bf16_bits(a))


def _normal(seed: int, sid: int, shape, std: float) -> np.ndarray:
    g = stream(seed, sid)
    return (g.standard_normal(int(np.prod(shape)), dtype=np.float32) * np.float32(std)).reshape(shape)


def _mixture_x(cfg: Config, seed: int, batch_seed: int) -> np.ndarray:
    """Hidden states from a Gaussian mixture: x = c_z + (noise_norm / sqrt(d)) * n.

    Centres c are unit-norm directions (normalised N(0, I) draws).  Labels z are
    drawn i.i.d., uniform over the centres when zipf_s == 0, else with weights
    proportional to (rank + 1) ** -zipf_s.  n ~ N(0, I), so the noise vector has
    norm close to noise_norm.
    """
    d, C = cfg.d, cfg.n_centroids
    g = _normal(seed, _S_CENTRES, (C, d), 1.0).astype(np.float64)
    centres = (g / np.linalg.norm(g, axis=1, keepdims=True)).astype(np.float32)
    if cfg.zipf_s > 0:
        w = (np.arange(1, C + 1, dtype=np.float64)) ** (-cfg.zipf_s)
    else:
        w = np.ones(C)
    w /= w.sum()
    labels = stream(batch_seed, _S_LABELS).choice(C, size=cfg.T, p=w)
    noise = _normal(batch_seed, _S_NOISE, (cfg.T, d), cfg.noise_norm / np.sqrt(d))
    return centres[labels] + noise


def make_layer_inputs(cfg: Config, seed: int = 0, batch_seed: int = 0,
                      with_dy: bool | None = None, parts=None) -> dict:
    """Draw one MoE layer's inputs for a config.

    Returns a dict of float32 arrays (bf16-representable where the config stores
    bf16): x [T,d], wr [E,d], w1 [E,f,d], w3 [E,f,d], w2 [E,d,f] and, when the
    workload has a backward pass, dy [T,d].  Weight layout is [expert, out, in].
    All weights are N(0, 1/d).  parts, when given, restricts the draw to the
    named tensors (each tensor's values do not depend on the others drawn).
    """
    T, d, E, f = cfg.T, cfg.d, cfg.E, cfg.f
    std = 1.0 / np.sqrt(d)
    if with_dy is None:
        with_dy = cfg.backward
    want = set(parts) if parts is not None else {"x", "wr", "w1", "w3", "w2"} | ({"dy"} if with_dy else set())
    out = {}
    if "wr" in want:
        out["wr"] = _normal(seed, _S_WR, (E, d), std)
    if "w1" in want:
        out["w1"] = _normal(seed, _S_W1, (E, f, d), std)
    if "w3" in want:
        out["w3"] = _normal(seed, _S_W3, (E, f, d), std)
    if "w2" in want:
        out["w2"] = _normal(seed, _S_W2, (E, d, f), std)
    if "x" in want:
        if cfg.x_kind == "normal":
            out["x"] = _normal(batch_seed, _S_X, (T, d), 1.0)
        elif cfg.x_kind == "mixture":
            out["x"] = _mixture_x(cfg, seed, batch_seed)
        else:
            raise ValueError(cfg.x_kind)
    if "dy" in want:
        out["dy"] = _normal(batch_seed, _S_DY, (T, d), 1.0)
    if cfg.act == "bf16":
        for key in ("x", "w1", "w3", "w2", "dy"):
            if key in out:
                out[key] = bf16_round(out[key])
    return out


def make_routing(T: int, E: int, k: int, seed: int = 0) -> np.ndarray:
    """Uniformly random k-subsets of the E experts, one per token, as int32 [T,k].

    Slot order inside a row is random too.  Used where a test needs routing
    that is independent of any router (e.g. closed forms for i.i.d. routing).
    """
    g = stream(seed, _S_ROUTE)
    keys = g.random((T, E))
    return np.argsort(keys, axis=1)[:, :k].astype(np.int32)
