"""fp64 definitions of the steps a Mamba block puts around the selective scan.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; it never imports
the product path.

Page "State Space Models (SSM)" (ultralytics.com glossary), section "Da S4 a
Mamba": each Mamba block wraps the selective SSM with a short convolution and
a SiLU gate, and Delta, B, C are functions of the current token.  The page gives no further detail; the plainest reading, kept
here and in the GPU path:

* ``causal_conv``: a depthwise causal convolution along the sequence, one
  K-tap filter and one bias per channel; tap k weighs the input k - (K - 1)
  tokens back (tap K - 1 is the current token); inputs before the first token
  are zero.  It runs over the channels that become x, B and C.
* ``silu(v) = v / (1 + exp(-v))`` after the convolution and on the gate.
* ``softplus(v) = log(1 + exp(v))`` turns the raw step plus its per-head bias
  into Delta >= 0.
* ``layer_in``: conv + SiLU, split into x [.., H, P], B and C [.., G, N], and
  Delta = softplus(dt_raw + dt_bias).
* ``layer_out``: the scan's y times silu(z), z being the gate's input.

Parity: pinned in tests/test_oracle_layer_pins.py (odd-part identities of
silu and softplus, softplus(0) = ln 2, unit-tap filters, causality, a
brute-force numpy.convolve comparison).
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if not isinstance(a, np.ndarray):   # torch tensor (fp32 / bf16): widen exactly
        import torch
        return a.detach().cpu().to(torch.float64).numpy()
    return a.astype(np.float64)


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def softplus(v):
    v = np.asarray(v, dtype=np.float64)
    return np.logaddexp(0.0, v)


def causal_conv(u, w, bias=None):
    """u [batch, L, Cd]; w [Cd, K]; bias [Cd] or None -> [batch, L, Cd]:
    out[b, t, c] = bias[c] + sum_k w[c, k] u[b, t - (K - 1) + k, c]."""
    u, w = _f64(u), _f64(w)
    batch, L, Cd = u.shape
    K = w.shape[1]
    out = np.zeros_like(u) if bias is None else np.broadcast_to(_f64(bias), u.shape).copy()
    for k in range(K):
        back = K - 1 - k
        if back >= L:
            continue
        out[:, back:, :] += w[None, None, :, k] * u[:, : L - back, :]
    return out


def layer_in(xbc, w, bias, dt_raw, dt_bias, H, P, G, N):
    """(x [b, L, H, P], B [b, L, G, N], C [b, L, G, N], dt [b, L, H]) in fp64."""
    v = silu(causal_conv(xbc, w, bias))
    batch, L, _ = v.shape
    x = v[:, :, : H * P].reshape(batch, L, H, P)
    Bm = v[:, :, H * P: H * P + G * N].reshape(batch, L, G, N)
    Cm = v[:, :, H * P + G * N:].reshape(batch, L, G, N)
    d = _f64(dt_raw)
    if dt_bias is not None:
        d = d + _f64(dt_bias)[None, None, :]
    return x, Bm, Cm, softplus(d)


def layer_out(y, z):
    """y * silu(z), elementwise."""
    return _f64(y) * silu(_f64(z))
