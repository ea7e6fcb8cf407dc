"""Error metrics shared by the parity tests (no arithmetic of the scan here).

gate:  max_i |g_i - r_i| / max_i |r_i| over one output tensor.  A per-element
ratio is ill-posed where the reference is near zero, so the gate normalises by
the tensor's largest magnitude; the per-element figure below is reported next
to it for information.
"""
from __future__ import annotations

import numpy as np


def _np64(a):
    if not isinstance(a, np.ndarray):
        a = a.detach().cpu().double().numpy()
    return np.asarray(a, dtype=np.float64)


def max_rel_err(got, ref) -> float:
    g, r = _np64(got), _np64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    scale = float(np.max(np.abs(r)))
    diff = float(np.max(np.abs(g - r)))
    if not np.isfinite(diff):
        return float("inf")
    return diff / scale if scale > 0 else diff


def elementwise_rel_err(got, ref) -> float:
    g, r = _np64(got), _np64(ref)
    if g.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(g - r) / (np.abs(r) + 1e-3 * rms + 1e-300)))
