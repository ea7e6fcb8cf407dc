"""Error metrics shared by the parity tests (no arithmetic of the scan here).

Two gates per output tensor, both at the test's tolerance (1e-4 for fp32
storage, 2e-2 for bf16 storage unless a test states a tighter one):

* ``max_rel_err``: max_i |g_i - r_i| / max_i |r_i|.  Normalised by the
  tensor's largest magnitude, so it is well posed near zero but blind to an
  error confined to entries much smaller than that maximum (with D ~ N(0, 1)
  the skip term D x sets the peak of y, and the scan terms are a few percent
  of it).
* ``elementwise_rel_err``: max_i |g_i - r_i| / m_i, where m_i is the sum of
  the magnitudes of every term that contributes to r_i.  The tests obtain m
  from the same oracle run on absolute-valued inputs (|x|, |B|, |C|, |D|,
  |initial state|; dt >= 0 and exp(dt A) > 0 already): every term of that
  recurrence is then non-negative, so its output is exactly the sum of the
  absolute values of the terms of r_i.  Each element is judged at the scale
  of its own terms, so an error in a term that is small next to the tensor's
  peak, or in one token among large ones, is seen.  A bound follows from the
  arithmetic: every term reaches the result through at most three roundings
  to the storage type with fp32 accumulation in between (the weighted
  operand of the chunk-state product, the chunk state S, the carried state
  as a matrix operand), and the result is rounded once more, so
  |g_i - r_i| <= (4 u + O(fp32)) m_i with u = 2^-9 for bf16 (about 7.8e-3)
  and u = 2^-24 for fp32.  The block around the scan rounds x, B and C once
  more before the scan (about 2 u more).  Without a magnitude the scale is
  |r_i| + rms(r).

The ratio against |r_i| + 1e-3 rms(r) is printed beside them for
information only: with bf16 operands it is dominated by entries near zero
whose terms cancel, and it has no useful bound.
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


def elementwise_rel_err(got, ref, scale=None) -> float:
    """max_i |g_i - r_i| / s_i, s_i = scale_i (the magnitude of r_i's terms)
    if given, else |r_i| + rms(r).  0 / 0 counts as 0."""
    g, r = _np64(got), _np64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    d = np.abs(g - r)
    if not np.all(np.isfinite(d)):
        return float("inf")
    if scale is None:
        s = np.abs(r) + float(np.sqrt(np.mean(r * r)))
    else:
        s = _np64(scale)
        assert s.shape == r.shape, (s.shape, r.shape)
        assert np.all(s >= 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d == 0, 0.0, d / s)
    return float(np.max(q))


def _floor_ratio(g, r, floor):
    rms = float(np.sqrt(np.mean(r * r)))
    d = np.abs(g - r)
    return float(np.max(d / (np.abs(r) + floor * rms + 1e-300)))


def gate(got, ref, tol: float, what: str = "", scale=None) -> tuple[float, float]:
    """Both gates at ``tol``; prints them and the 1e-3-floor ratio.
    Returns (max_rel_err, elementwise_rel_err)."""
    g, r = _np64(got), _np64(ref)
    e_max = max_rel_err(g, r)
    e_ew = elementwise_rel_err(g, r, scale)
    e_info = _floor_ratio(g, r, 1e-3) if g.size else 0.0
    kind = "terms" if scale is not None else "|r|+rms"
    print(f"  {what}: max_rel {e_max:.3e}  elementwise[{kind}] {e_ew:.3e}  "
          f"(vs |r|+1e-3 rms: {e_info:.3e})", flush=True)
    assert e_max <= tol, (what, "max_rel_err", e_max, tol)
    assert e_ew <= tol, (what, "elementwise_rel_err", e_ew, tol)
    return e_max, e_ew
