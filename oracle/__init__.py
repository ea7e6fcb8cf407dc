"""fp64 CPU oracle for the selective SSM with a scalar decay per head.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``mamba_ssd_scan_02_amd``) never imports it, and it never imports the
product path.

Contents
--------
* ``ssd_oracle.c``   the plain sequential fp64 recurrence (built with gcc into
  ``libssd_oracle.so``), wrapped here through ctypes: ``forward`` and ``step``.
* ``stages.py``      fp64 NumPy definitions of the four chunk stages, used only
  to localise a GPU discrepancy to one stage; they are checked against the
  recurrence, never the other way round.

Parity status of each function is listed in its docstring; every function here
is pinned by a CPU test under ``tests/`` (see ``tests/test_oracle_pins.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "ssd_oracle.c"
_LIB = _HERE / "libssd_oracle.so"

IN_F32 = 0
IN_BF16 = 1

_lib = None


def build(verbose: bool = False) -> Path:
    """Compile ``ssd_oracle.c`` with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", str(_LIB) + ".tmp", str(_SRC), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(str(_LIB) + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB.exists():
        build()
    lib = ctypes.CDLL(str(_LIB))
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_abi_version.restype = i32
    lib.oracle_max_threads.restype = i32
    lib.oracle_ssd_forward.restype = i32
    lib.oracle_ssd_forward.argtypes = [i64, i64, i64, i64, i64, i64, i32,
                                       vp, vp, vp, vp, vp, vp, vp,
                                       vp, i64, i64, i64, vp, vp]
    lib.oracle_ssm_step.restype = i32
    lib.oracle_ssm_step.argtypes = [i64, i64, i64, i64, i64, i32,
                                    vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_ssd_forward_ex.restype = i32
    lib.oracle_ssd_forward_ex.argtypes = lib.oracle_ssd_forward.argtypes + [i32]
    lib.oracle_ssm_step_ex.restype = i32
    lib.oracle_ssm_step_ex.argtypes = lib.oracle_ssm_step.argtypes + [i32]
    _lib = lib
    return lib


def _as_storage(a):
    """Return (contiguous numpy array, kind).  Accepts numpy float32, numpy
    uint16 holding bf16 bit patterns, or a CPU torch tensor (float32/bfloat16)."""
    if a is None:
        return None, None
    if not isinstance(a, np.ndarray):  # torch tensor
        import torch
        t = a.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), IN_BF16
        return t.to(torch.float32).numpy(), IN_F32
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a), IN_BF16
    return np.ascontiguousarray(a, dtype=np.float32), IN_F32


def _f32(a):
    if a is None:
        return None
    arr, kind = _as_storage(a)
    if kind != IN_F32:
        raise TypeError("expected an fp32 array")
    return arr


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def forward(x, dt, A, B, C, D=None, init=None, ngroups=None, bh=None, t_range=None, zoh=False):
    """Sequential fp64 recurrence over whole sequences.

    Shapes: x [batch, L, H, P]; dt [batch, L, H]; A [H]; B, C [batch, L, G, N];
    D [H] or None; init [batch, H, P, N] or None.  x, B, C share one storage
    type (fp32, or bf16 given as uint16 bits / torch bfloat16).

    ``bh`` is a list of (b, h) pairs (default: all, b-major); ``t_range`` limits
    which tokens of y are returned (the recurrence always starts at t = 0).

    ``zoh`` selects the exact zero-order-hold input weight expm1(dt A) / A in
    place of dt (see ssd_oracle.c).

    Returns ``(y_sel [n_bh, T, P] float64, final_sel [n_bh, P, N] float64)``.
    Parity: pinned (water tank, convolution form, materialised semiseparable
    matrix, linear-attention special case, limits, split invariance; the
    zero-order hold by the convolution demo, its steady state and its
    small-step limit).
    """
    lib = _load()
    xs, kind = _as_storage(x)
    bs, kb = _as_storage(B)
    cs, kc = _as_storage(C)
    if not (kind == kb == kc):
        raise TypeError("x, B and C must share one storage type")
    dts, As, Ds, inits = _f32(dt), _f32(A), _f32(D), _f32(init)
    batch, L, H, P = xs.shape
    G, N = bs.shape[2], bs.shape[3]
    if ngroups is not None and ngroups != G:
        raise ValueError("ngroups does not match B")
    assert dts.shape == (batch, L, H) and As.shape == (H,)
    assert bs.shape == (batch, L, G, N) and cs.shape == (batch, L, G, N)
    if Ds is not None:
        assert Ds.shape == (H,)
    if inits is not None:
        assert inits.shape == (batch, H, P, N)
    if bh is None:
        bh = [(b, h) for b in range(batch) for h in range(H)]
    bh_arr = np.ascontiguousarray(np.asarray(bh, dtype=np.int64).reshape(-1, 2))
    t0, t1 = (0, L) if t_range is None else (int(t_range[0]), int(t_range[1]))
    n = bh_arr.shape[0]
    y = np.empty((n, t1 - t0, P), dtype=np.float64)
    fin = np.empty((n, P, N), dtype=np.float64)
    rc = lib.oracle_ssd_forward_ex(batch, L, H, P, N, G, kind, _ptr(xs), _ptr(dts), _ptr(As),
                                   _ptr(bs), _ptr(cs), _ptr(Ds), _ptr(inits),
                                   _ptr(bh_arr), n, t0, t1, _ptr(y), _ptr(fin), int(bool(zoh)))
    if rc != 0:
        raise ValueError(f"oracle_ssd_forward failed with {rc}")
    return y, fin


def forward_full(x, dt, A, B, C, D=None, init=None, zoh=False):
    """``forward`` over every (b, h), reshaped to y [batch, L, H, P] and
    final [batch, H, P, N] (float64)."""
    xs, _ = _as_storage(x)
    batch, L, H, P = xs.shape
    y_sel, fin = forward(x, dt, A, B, C, D, init, zoh=zoh)
    y = y_sel.reshape(batch, H, L, P).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(y), fin.reshape(batch, H, P, -1)


def step(state, x_t, dt_t, A, B_t, C_t, D=None, zoh=False):
    """One decode step of the same recurrence.  ``state`` [batch, H, P, N]
    float64 is updated in place; returns y_t [batch, H, P] float64.
    Parity: pinned (equals ``forward`` run one token at a time, water tank)."""
    lib = _load()
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise TypeError("state must be a C-contiguous float64 array")
    xs, kind = _as_storage(x_t)
    bs, kb = _as_storage(B_t)
    cs, kc = _as_storage(C_t)
    if not (kind == kb == kc):
        raise TypeError("x_t, B_t and C_t must share one storage type")
    dts, As, Ds = _f32(dt_t), _f32(A), _f32(D)
    batch, H, P, N = state.shape
    G = bs.shape[1]
    assert xs.shape == (batch, H, P) and dts.shape == (batch, H)
    assert bs.shape == (batch, G, N) and cs.shape == (batch, G, N)
    y = np.empty((batch, H, P), dtype=np.float64)
    rc = lib.oracle_ssm_step_ex(batch, H, P, N, G, kind, _ptr(state), _ptr(xs), _ptr(dts),
                                _ptr(As), _ptr(bs), _ptr(cs), _ptr(Ds), _ptr(y), int(bool(zoh)))
    if rc != 0:
        raise ValueError(f"oracle_ssm_step failed with {rc}")
    return y


def threads() -> int:
    """Number of OpenMP threads an oracle call runs on."""
    return int(_load().oracle_max_threads())
