"""Helpers shared by the GPU parity tests: device transfer and the error metric."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances.  fp32 workloads: 1e-4; bf16 workloads: 2e-2 for everything
# downstream of the expert path; the router's own outputs are fp32 in every
# workload and are held to 1e-4.
TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL_ROUTER = 1e-4


def act_torch(cfg_act: str) -> torch.dtype:
    return torch.bfloat16 if cfg_act == "bf16" else torch.float32


def dev(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Upload exactly: values are bf16-representable where dtype is bf16."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda", dtype=dtype).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def rel_err(gpu, ref) -> float:
    """Relative error of a tensor: the largest normwise relative error of its
    rows (last axis), max_r ||g_r - o_r||_inf / max(||o_r||_inf, rms(o)).

    Normwise per row because an entry produced by a dot product carries an
    error proportional to the size of the terms summed, not to its own value:
    elementwise ratios are undefined at cancellation zeros and blow up in
    heavy-tailed rows.  The tensor's RMS floors rows of negligible size."""
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if o.size == 0:
        return 0.0
    if o.ndim == 0:
        g, o = g.reshape(1, 1), o.reshape(1, 1)
    elif o.ndim == 1:
        g, o = g.reshape(-1, 1), o.reshape(-1, 1)
    else:
        g, o = g.reshape(-1, o.shape[-1]), o.reshape(-1, o.shape[-1])
    rms = float(np.sqrt(np.mean(o * o)))
    if rms == 0.0:
        return float(np.abs(g).max())
    num = np.abs(g - o).max(axis=1)
    den = np.maximum(np.abs(o).max(axis=1), rms)
    return float((num / den).max())


def per_slice_err(gpu, ref) -> float:
    """rel_err per leading-axis slice (per expert for weight gradients)."""
    return max((rel_err(gpu[i], ref[i]) for i in range(ref.shape[0])), default=0.0)


# ---------------------------------------------------------------------------
# Parity of float outputs against the exact (fp64, unrounded) oracle.
#
# Every element of every float output must lie within C_BOUND times its
# first-order error bound B (oracle.layer_error_bounds: the rounding of the
# stored activations and the fp32 sums, carried through the layer from the
# exact operands; Higham, Accuracy and Stability of Numerical Algorithms,
# Sec. 3.1).  C_BOUND = 2 leaves room for the second-order terms that the
# first-order bound drops.  Beside it, the workload tolerance (1e-4 fp32,
# 2e-2 bf16) holds for the row-normwise error of every output outside
# `bound_only` (outputs that cancel so much that a bf16-storage computation
# misses 2e-2 there by rounding alone: the logit gradient, and the expert
# weight gradients of the clustered-input workloads).  Rows are the last axis;
# the expert weight gradients are taken per expert slice.
# Both the elementwise error (|g-o| / max(|o|, rms)) and the row-normwise one
# are printed.
# ---------------------------------------------------------------------------

C_BOUND = 2.0
SLICED = ("dw1", "dw3", "dw2")   # per expert: [E, out, in] -> one [out, in] slice each


def a13_err(gpu, ref) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms(o)) over one tensor."""
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    if rms == 0.0:
        return float(np.abs(g).max())
    return float((np.abs(g - o) / np.maximum(np.abs(o), rms)).max())


def bound_ratio(gpu, ref, bound) -> float:
    """max_i |g_i - o_i| / B_i (0/0 counts as 0)."""
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    b = np.asarray(bound, dtype=np.float64)
    assert g.shape == o.shape == b.shape, (g.shape, o.shape, b.shape)
    if o.size == 0:
        return 0.0
    diff = np.abs(g - o)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(diff == 0.0, 0.0, diff / b)
    return float(np.nan_to_num(r, nan=np.inf, posinf=np.inf).max())


def check_floats(label, got: dict, exact: dict, bounds: dict, tol: float, bound_only=()):
    """Hold every tensor in `got` to the exact oracle values and their bounds;
    prints one line per tensor and asserts at the end (all tensors reported)."""
    fails = []
    for key, g in got.items():
        o, b = exact[key], bounds[key]
        sl = key in SLICED
        e13 = (max((a13_err(g[i], o[i]) for i in range(o.shape[0])), default=0.0) if sl
               else a13_err(g, o))
        ern = per_slice_err(g, o) if sl else rel_err(g, o)
        rb = bound_ratio(g, o, b)
        only = key in bound_only
        print(f"[{label}] {key:8s} elementwise {e13:.2e}  row-normwise {ern:.2e}  "
              f"max|err|/B {rb:.3f}{'  (bound only)' if only else ''}", flush=True)
        if not rb <= C_BOUND:
            fails.append((key, "bound", rb))
        if not only and not ern <= tol:
            fails.append((key, "tolerance", ern))
    assert not fails, f"{label}: {fails}"
