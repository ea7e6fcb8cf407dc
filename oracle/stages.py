"""fp64 NumPy definitions of the four chunk stages of the block algorithm.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).  These functions exist to
tell which stage of a GPU pipeline disagrees with the recurrence oracle; they
are checked against ``oracle.forward`` for many chunk sizes and are never used
as the authority on the final result.

The block algorithm: the sequence is cut into contiguous blocks; inside a
block the output is computed in the quadratic, attention-like form, and only a
summary state is carried from one block to the next (page "Mamba-2 (2024): SSM
e attention sono la stessa cosa", paithon.it, section "Il trucco a blocchi";
page "Architektury Mamba-2, State Space Models i liniowa atencja...",
tech.tersel.eu, section "Rewolucja Mamba-2 i teoria State Space Duality SSD").
The quadratic form inside a block is masked attention without softmax where
the interaction of positions i >= j is weighted by how much of j survived until
i (page "State Space Model", book.paithon.it, section "Due strade, una meta").

Unrolling the recurrence of ``oracle.forward`` over one block of Q tokens
(t = cQ + i, a_t = exp(dt_t A_h), Acs[i] = sum_{k<=i} dt_k A_h) gives

    S_c   = sum_j exp(Acs[last] - Acs[j]) dt_j  x_j (outer) B_j        (P x N)
    H_0   = init,  H_{c+1} = exp(Acs[last]) H_c + S_c,  final = H_nc
    y_i   = sum_{j<=i} (C_i . B_j) exp(Acs[i] - Acs[j]) dt_j x_j
            + exp(Acs[i]) H_c C_i + D x_i

which is what the four functions below compute, in that order.
Parity: pinned against the recurrence for chunk sizes 1, 7, 64 and L.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if not isinstance(a, np.ndarray):
        a = a.detach().cpu().float().numpy()
    return np.asarray(a, dtype=np.float64)


def n_chunks(L: int, Q: int) -> int:
    return (L + Q - 1) // Q


def chunk_cumsum(dt, A, Q):
    """Acs [batch, H, nc, Q]: inclusive prefix over each block of dt * A_h.
    Positions past the end of the sequence (last block only) repeat the last
    valid value, i.e. they add no decay."""
    dt, A = _f64(dt), _f64(A)
    batch, L, H = dt.shape
    nc = n_chunks(L, Q)
    pad = np.zeros((batch, nc * Q, H))
    pad[:, :L] = dt * A[None, None, :]
    blocks = pad.reshape(batch, nc, Q, H)
    return np.cumsum(blocks, axis=2).transpose(0, 3, 1, 2).copy()


def _blocked(a, L, Q):
    """Zero-pad the token axis (axis 1) to a multiple of Q and split it."""
    nc = n_chunks(L, Q)
    shape = (a.shape[0], nc * Q) + a.shape[2:]
    out = np.zeros(shape)
    out[:, :L] = a
    return out.reshape((a.shape[0], nc, Q) + a.shape[2:])


def _group_of_head(H, G):
    return np.arange(H) // (H // G)


def chunk_state(x, dt, B, Acs, Q):
    """S [batch, H, nc, P, N]: each block's end state, starting from zero."""
    x, dt, B = _f64(x), _f64(dt), _f64(B)
    batch, L, H, P = x.shape
    G = B.shape[2]
    xb = _blocked(x, L, Q)                                    # b c j h p
    dtb = _blocked(dt, L, Q)                                  # b c j h
    Bb = _blocked(B, L, Q)[:, :, :, _group_of_head(H, G)]     # b c j h n
    acs = Acs.transpose(0, 2, 3, 1)                           # b c j h
    w = np.exp(acs[:, :, -1:, :] - acs) * dtb                 # b c j h
    return np.einsum("bcjh,bcjhp,bcjhn->bhcpn", w, xb, Bb)


def state_passing(S, Acs, init=None):
    """Hin [batch, H, nc, P, N] (state entering each block) and final state."""
    batch, H, nc, P, N = S.shape
    h = np.zeros((batch, H, P, N)) if init is None else _f64(init).copy()
    Hin = np.empty_like(S)
    for c in range(nc):
        Hin[:, :, c] = h
        h = np.exp(Acs[:, :, c, -1])[:, :, None, None] * h + S[:, :, c]
    return Hin, h


def run_states(S, Acs, K):
    """First level of the two-level recurrence between blocks, runs of K
    blocks (run r = blocks rK .. min(rK + K, nc) - 1).  Two steps of the
    recurrence h <- a h + s merge into one step of the same kind (the
    parallel scan of page "State Space Model", section "Dai sistemi dinamici
    a Mamba"), so each run is scanned from a zero state on its own:
        T[c]    = the state after block c from zero at its run's start
        lam[c]  = summed decay (natural log) of the run's blocks before c
        rdec[r] = summed decay of run r's blocks.
    Returns (T [batch, H, nc, P, N], lam [batch, H, nc], rdec [batch, H, nruns])."""
    batch, H, nc, P, N = S.shape
    nruns = (nc + K - 1) // K
    T = np.empty_like(S, dtype=np.float64)
    lam = np.zeros((batch, H, nc))
    rdec = np.zeros((batch, H, nruns))
    for r in range(nruns):
        h = np.zeros((batch, H, P, N))
        ls = np.zeros((batch, H))
        for c in range(r * K, min(r * K + K, nc)):
            lam[:, :, c] = ls
            h = np.exp(Acs[:, :, c, -1])[:, :, None, None] * h + S[:, :, c]
            T[:, :, c] = h
            ls = ls + Acs[:, :, c, -1]
        rdec[:, :, r] = ls
    return T, lam, rdec


def run_passing(T, rdec, K, init=None):
    """Second level: the chain over runs, Hr[0] = init (or 0),
    Hr[r + 1] = exp(rdec[r]) Hr[r] + T[last block of run r]; returns
    (Hr [batch, H, nruns, P, N], final state)."""
    batch, H, nc, P, N = T.shape
    nruns = rdec.shape[2]
    h = np.zeros((batch, H, P, N)) if init is None else _f64(init).copy()
    Hr = np.empty((batch, H, nruns, P, N))
    for r in range(nruns):
        Hr[:, :, r] = h
        last = min(r * K + K, nc) - 1
        h = np.exp(rdec[:, :, r])[:, :, None, None] * h + T[:, :, last]
    return Hr, h


def runs_entering_states(T, Hr, lam, K):
    """The state entering each block from the two levels: Hr[r] at a run's
    first block, T[c - 1] + exp(lam[c]) Hr[r] past it."""
    batch, H, nc, P, N = T.shape
    Hin = np.empty((batch, H, nc, P, N))
    for c in range(nc):
        r = c // K
        if c % K == 0:
            Hin[:, :, c] = Hr[:, :, r]
        else:
            Hin[:, :, c] = T[:, :, c - 1] + np.exp(lam[:, :, c])[:, :, None, None] * Hr[:, :, r]
    return Hin


def chunk_scan(x, dt, B, C, Acs, Hin, D, Q):
    """y [batch, L, H, P]: masked quadratic form inside each block plus the
    carried-state term and the D skip term."""
    x, dt, B, C = _f64(x), _f64(dt), _f64(B), _f64(C)
    batch, L, H, P = x.shape
    G = B.shape[2]
    gh = _group_of_head(H, G)
    xb = _blocked(x, L, Q)
    dtb = _blocked(dt, L, Q)
    Bb = _blocked(B, L, Q)[:, :, :, gh]                       # b c j h n
    Cb = _blocked(C, L, Q)[:, :, :, gh]                       # b c i h n
    acs = Acs.transpose(0, 2, 3, 1)                           # b c i h
    CB = np.einsum("bcihn,bcjhn->bchij", Cb, Bb)
    diff = acs.transpose(0, 1, 3, 2)[..., :, None] - acs.transpose(0, 1, 3, 2)[..., None, :]
    mask = np.tril(np.ones((Q, Q), dtype=bool))
    decay = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)   # b c h i j
    Wm = CB * decay * dtb.transpose(0, 1, 3, 2)[:, :, :, None, :]
    y = np.einsum("bchij,bcjhp->bcihp", Wm, xb)
    y += np.exp(acs)[..., None] * np.einsum("bcihn,bhcpn->bcihp", Cb, Hin)
    if D is not None:
        y += _f64(D)[None, None, None, :, None] * xb
    return y.reshape(batch, -1, H, P)[:, :L]


def forward(x, dt, A, B, C, D, init, Q):
    """The four stages chained: returns (y, final, Acs, S, Hin)."""
    Acs = chunk_cumsum(dt, A, Q)
    S = chunk_state(x, dt, B, Acs, Q)
    Hin, final = state_passing(S, Acs, init)
    y = chunk_scan(x, dt, B, C, Acs, Hin, D, Q)
    return y, final, Acs, S, Hin
