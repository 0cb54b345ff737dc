"""The five workload shapes of the MoE-layer hot path.

Shapes follow the small-model study of "MoE Pretraining: Parallelism Layout
Changes the Model, Not Quality" (Methodology, Models and Data table: 16 SwiGLU
experts of width 256, top-4, global batch 32 x 512 tokens) and two larger
layers in the spirit of "Expert Coupling in MoE Pretraining" (Abstract: top-2
and top-6 routing; Table I: EP8 and EP16 placements).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    T: int            # tokens on this GPU
    d: int            # model width
    E: int            # experts
    f: int            # expert FFN width
    k: int            # experts per token
    act: str          # "f32" or "bf16": X, W1/W3/W2, Y, dY, dX storage type
    backward: bool    # whether the workload runs the backward pass
    x_kind: str       # "normal" or "mixture"
    n_centroids: int = 0
    noise_norm: float = 0.0      # norm of the noise vector around a centre
    zipf_s: float = 0.0          # 0 -> uniform mixture weights
    lb_groups: Tuple[int, ...] = (1,)
    plan_groups: Tuple[int, ...] = ()
    description: str = field(default="", compare=False)

    @property
    def R(self) -> int:
        return self.T * self.k

    def gemm_flops_fwd(self) -> int:
        # x_perm @ W1^T, x_perm @ W3^T and h @ W2^T: three R x d x f products
        return 6 * self.R * self.d * self.f

    def gemm_flops_bwd(self) -> int:
        # dgrad (dh, dx_perm through W1 and W3) and wgrad (dW1, dW3, dW2)
        return 12 * self.R * self.d * self.f


# Zipf exponent of the 64-centroid mixture, chosen so that the 20 most frequent
# expert pairs (about 1% of the C(64,2) pairs) carry about 40% of the tokens'
# top-2 selections.  tests/test_synth.py checks that property.
MIXTURE64_ZIPF_S = 0.85

CONFIGS = {
    "c1": Config(
        "c1", T=2048, d=256, E=8, f=256, k=2, act="f32", backward=False,
        x_kind="normal",
        description="tiny fp32 layer, forward only"),
    "c2": Config(
        "c2", T=16384, d=256, E=16, f=256, k=4, act="bf16", backward=True,
        x_kind="normal", lb_groups=(1, 2, 4, 8),
        description="small-model layer, 32x512 tokens, 16 experts, top-4"),
    "c3": Config(
        "c3", T=16384, d=256, E=64, f=64, k=4, act="bf16", backward=True,
        x_kind="mixture", n_centroids=32, noise_norm=0.3, zipf_s=0.0,
        description="fine-grained experts, 32-centroid mixture"),
    "c4": Config(
        "c4", T=16384, d=2048, E=64, f=1024, k=2, act="bf16", backward=True,
        x_kind="mixture", n_centroids=64, noise_norm=0.3,
        zipf_s=MIXTURE64_ZIPF_S, plan_groups=(8,),
        description="mid-size layer, top-2, correlated 64-centroid mixture"),
    "c5": Config(
        "c5", T=16384, d=2048, E=64, f=1024, k=6, act="bf16", backward=True,
        x_kind="mixture", n_centroids=64, noise_norm=0.3,
        zipf_s=MIXTURE64_ZIPF_S, plan_groups=(8, 16),
        description="mid-size layer, top-6, correlated 64-centroid mixture"),
}


def get_config(name: str, **overrides) -> Config:
    """Return a named config, optionally with fields replaced (e.g. a smaller T)."""
    base = CONFIGS[name.lower()]
    if not overrides:
        return base
    fields = {f: getattr(base, f) for f in base.__dataclass_fields__}
    fields.update(overrides)
    return Config(**fields)
