"""Shared helpers for the GPU tests: run the HIP path on CPU-held inputs and
compare with the oracle.  No arithmetic of the scan lives here.

Outputs and workspaces handed to the library are *guarded*: each sits inside a
larger allocation whose GUARD_BYTES on either side hold a canary byte pattern,
and its own bytes start as 0xFF (NaN in fp32 and bf16).  After the call the
guard bands must be intact (no store landed outside the output) and, for
outputs, every element must have been written (a NaN left behind fails the
parity check); a NaN-filled workspace makes any read of a workspace byte that
was never written show up in the results."""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}

GUARD_BYTES = 1 << 16
CANARY = 0xA5
POISON = 0xFF


def to_gpu(inp: dict) -> dict:
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


class Guarded:
    """A contiguous device tensor of ``shape`` inside canary guard bands."""

    def __init__(self, shape, dtype, fill=POISON, device="cuda"):
        es = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        g = GUARD_BYTES // es
        self.buf = torch.empty(n + 2 * g, dtype=dtype, device=device)
        self.buf.view(torch.uint8).fill_(CANARY)
        self.t = self.buf[g:g + n].view(*shape)
        if fill is not None:
            self.t.view(torch.uint8).fill_(fill)
        self.nbytes = n * es

    def intact(self) -> bool:
        u = self.buf.view(torch.uint8)
        return bool((u[:GUARD_BYTES] == CANARY).all()) and \
            bool((u[GUARD_BYTES + self.nbytes:] == CANARY).all())


def gpu_forward(inp: dict, chunk: int, **kw):
    """ssd_forward through the binding with guarded, NaN-filled y and final
    state and a NaN-poisoned, guarded workspace."""
    import mamba_ssd_scan_02_amd as ssd
    g = to_gpu(inp)
    x = g["x"]
    batch, L, H, P = x.shape
    G, N = g["B"].shape[2], g["B"].shape[3]
    yb = Guarded(tuple(x.shape), x.dtype)
    fb = Guarded((batch, H, P, N), torch.float32)
    need = ssd.workspace_bytes(batch, L, H, P, N, G, chunk, x.dtype)
    wb = Guarded((need,), torch.uint8)
    y, fin = ssd.ssd_forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g.get("D"), chunk,
                             g.get("init"), y=yb.t, final_state=fb.t, workspace=wb.t, **kw)
    torch.cuda.synchronize()
    assert yb.intact(), "a store landed outside y"
    assert fb.intact(), "a store landed outside final_state"
    assert wb.intact(), "a store landed outside the workspace"
    return y, fin


def oracle_forward(inp: dict, bh=None, t_range=None, zoh=False):
    import oracle
    return oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                          inp.get("init"), bh=bh, t_range=t_range, zoh=zoh)


def abs_inputs(inp: dict) -> dict:
    """The inputs with x, B, C, D and the initial state replaced by their
    absolute values (exact in either storage type); dt and A unchanged."""
    out = dict(inp)
    for k in ("x", "B", "C", "D", "init"):
        if out.get(k) is not None:
            out[k] = out[k].abs()
    return out


def oracle_forward_scaled(inp: dict, bh=None, t_range=None, zoh=False):
    """(y, final) of the oracle and their magnitudes (the oracle on
    abs_inputs: the sum of the absolute values of every term of each
    output), the two runs side by side in two host threads."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(2) as ex:
        fv = ex.submit(oracle_forward, inp, bh, t_range, zoh)
        fm = ex.submit(oracle_forward, abs_inputs(inp), bh, t_range, zoh)
        (y, f), (ym, fm_) = fv.result(), fm.result()
    return y, f, ym, fm_


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
