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
