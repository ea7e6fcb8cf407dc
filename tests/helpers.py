"""Shared helpers for the GPU tests: run the HIP path on CPU-held inputs and
compare with the oracle.  No arithmetic of the scan lives here."""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_gpu(inp: dict) -> dict:
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_forward(inp: dict, chunk: int, **kw):
    import mamba_ssd_scan_02_amd as ssd
    g = to_gpu(inp)
    y, fin = ssd.ssd_forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g.get("D"), chunk,
                             g.get("init"), **kw)
    torch.cuda.synchronize()
    return y, fin


def oracle_forward(inp: dict, bh=None, t_range=None, zoh=False):
    import oracle
    return oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                          inp.get("init"), bh=bh, t_range=t_range, zoh=zoh)


def select_y(y: torch.Tensor, bh, t_range=None) -> np.ndarray:
    """Rows of y [batch, L, H, P] for the (b, h) list, as [n, T, P] float64."""
    L = y.shape[1]
    t0, t1 = (0, L) if t_range is None else t_range
    return np.stack([y[b, t0:t1, h].float().cpu().numpy().astype(np.float64) for b, h in bh])


def select_state(s: torch.Tensor, bh) -> np.ndarray:
    return np.stack([s[b, h].float().cpu().numpy().astype(np.float64) for b, h in bh])


def all_pairs(batch, H):
    return [(b, h) for b in range(batch) for h in range(H)]


def sample_pairs(batch, H, n, seed=0):
    rng = np.random.default_rng(seed)
    pairs = all_pairs(batch, H)
    idx = rng.choice(len(pairs), size=min(n, len(pairs)), replace=False)
    # always include the first and the last pair
    chosen = sorted(set(int(i) for i in idx) | {0, len(pairs) - 1})
    return [pairs[i] for i in chosen]


def say(msg: str):
    print(msg, flush=True)
