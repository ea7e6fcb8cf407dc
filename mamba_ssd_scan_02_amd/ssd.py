"""Python binding of libssd_mi355x.so (the C ABI in include/ssd_mi355x.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and torch's current HIP stream are handed to
the C entry points, and outputs / workspace are allocated with torch.  Every
step of the computation runs in the library's gfx950 kernels; if the library
is missing or was built without GPU support the first call raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
_LIB_PATH = _PKG / "libssd_mi355x.so"

DTYPE_F32 = 0
DTYPE_BF16 = 1

# The SSD_ABI_VERSION this binding was written against; load() refuses a
# library that reports another one (a stale build).
ABI_VERSION = 8

_STATUS_OK = 0

_lib = None


class SSDError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_str(status)})")


def library_path() -> Path:
    return _LIB_PATH


def load():
    """Load the shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m mamba_ssd_scan_02_amd.csrc.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(str(_LIB_PATH))
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.ssd_abi_version.restype = i32
    lib.ssd_abi_version.argtypes = []
    lib.ssd_status_str.restype = ctypes.c_char_p
    lib.ssd_status_str.argtypes = [i32]
    lib.ssd_forward_workspace_bytes.restype = sz
    lib.ssd_forward_workspace_bytes.argtypes = [i64] * 7 + [i32]
    lib.ssd_forward.restype = i32
    lib.ssd_forward.argtypes = [i64] * 7 + [i32] + [vp] * 9 + [vp, sz, vp]
    lib.ssd_forward_zoh.restype = i32
    lib.ssd_forward_zoh.argtypes = lib.ssd_forward.argtypes
    lib.ssd_forward_gated.restype = i32
    lib.ssd_forward_gated.argtypes = [i64] * 7 + [i32] + [vp] * 10 + [vp, sz, vp]
    lib.ssd_forward_noalloc.restype = i32
    lib.ssd_forward_noalloc.argtypes = [i64] * 7 + [i32] + [vp] * 9 + [vp]
    lib.ssm_step.restype = i32
    lib.ssm_step.argtypes = [i64] * 5 + [i32] + [vp] * 8 + [vp]
    lib.ssm_step_zoh.restype = i32
    lib.ssm_step_zoh.argtypes = lib.ssm_step.argtypes
    lib.ssd_chunk_cumsum.restype = i32
    lib.ssd_chunk_cumsum.argtypes = [i64] * 4 + [vp] * 4 + [vp]
    lib.ssd_chunk_cumsum_zoh.restype = i32
    lib.ssd_chunk_cumsum_zoh.argtypes = lib.ssd_chunk_cumsum.argtypes
    lib.ssd_chunk_state.restype = i32
    lib.ssd_chunk_state.argtypes = [i64] * 7 + [i32] + [vp] * 5 + [vp]
    lib.ssd_chunk_cumsum_state.restype = i32
    lib.ssd_chunk_cumsum_state.argtypes = [i64] * 7 + [i32] + [vp] * 7 + [vp]
    lib.ssd_state_passing.restype = i32
    lib.ssd_state_passing.argtypes = [i64] * 6 + [i32] + [vp] * 5 + [vp]
    lib.ssd_state_scan.restype = i32
    lib.ssd_state_scan.argtypes = [i64] * 7 + [i32] + [vp] * 7 + [vp]
    lib.ssd_chunk_scan.restype = i32
    lib.ssd_chunk_scan.argtypes = [i64] * 7 + [i32] + [vp] * 8 + [vp]
    lib.ssd_state_passing_seg_workspace_bytes.restype = sz
    lib.ssd_state_passing_seg_workspace_bytes.argtypes = [i64] * 5
    lib.ssd_state_passing_seg.restype = i32
    lib.ssd_state_passing_seg.argtypes = [i64] * 7 + [i32] + [vp] * 6 + [sz, vp]
    lib.ssd_forward_run_chunks.restype = i64
    lib.ssd_forward_run_chunks.argtypes = [i64] * 7 + [i32]
    lib.ssd_chunk_state_runs.restype = i32
    lib.ssd_chunk_state_runs.argtypes = [i64] * 7 + [i32, i64] + [vp] * 9 + [vp]
    lib.ssd_run_passing.restype = i32
    lib.ssd_run_passing.argtypes = [i64] * 6 + [i32, i64] + [vp] * 5 + [vp]
    lib.ssd_chunk_scan_runs.restype = i32
    lib.ssd_chunk_scan_runs.argtypes = [i64] * 7 + [i32, i64] + [vp] * 10 + [vp]
    lib.ssd_layer_in.restype = i32
    lib.ssd_layer_in.argtypes = [i64] * 7 + [i32] + [vp] * 9 + [vp]
    lib.ssd_layer_out.restype = i32
    lib.ssd_layer_out.argtypes = [i64, i32, vp, vp, vp, vp]

    got = int(lib.ssd_abi_version())
    if got != ABI_VERSION:
        raise RuntimeError(f"{_LIB_PATH} reports ABI version {got}, this binding needs "
                           f"{ABI_VERSION}: rebuild the library")
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().ssd_status_str(int(status)).decode()


def abi_version() -> int:
    return int(load().ssd_abi_version())


# --------------------------------------------------------------------------
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported storage dtype {t.dtype} (bf16 or fp32)")


def _dev(t, name, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn, status):
    if status != _STATUS_OK:
        raise SSDError(fn, status)


def n_chunks(seqlen: int, chunk: int) -> int:
    return (seqlen + chunk - 1) // chunk


def workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32)
    return int(load().ssd_forward_workspace_bytes(batch, seqlen, nheads, headdim, dstate, ngroups,
                                                  chunk, code))


def workspace_regions(batch, seqlen, nheads, headdim, dstate, chunk, dtype):
    """Byte offsets and element counts of cs, dtc, S, Hin inside the workspace
    (the layout documented at ssd_forward_workspace_bytes; S and Hin in the
    storage type)."""
    nc = n_chunks(seqlen, chunk)
    es = 2 if dtype == torch.bfloat16 else 4
    up = lambda v: (v + 255) // 256 * 256
    rows = batch * nheads * nc * chunk
    states = batch * nheads * nc * headdim * dstate
    off_dtc = up(rows * 4)
    off_S = off_dtc + up(rows * 4)
    off_H = off_S + up(states * es)
    return dict(cs=(0, rows), dtc=(off_dtc, rows), S=(off_S, states), Hin=(off_H, states),
                total=off_H + up(states * es))


def ssd_forward(x, dt, A, B, C, D=None, chunk=256, init_state=None, *, y=None,
                final_state=None, workspace=None, return_final_state=True, zoh=False, z=None):
    """Whole-sequence SSD forward on the GPU.

    x [batch, L, H, P] (bf16 | fp32); dt [batch, L, H] fp32; A [H] fp32;
    B, C [batch, L, G, N] (x's dtype); D [H] fp32 or None;
    init_state [batch, H, P, N] fp32 or None.
    Returns (y [batch, L, H, P] in x's dtype, final_state [batch, H, P, N] fp32
    or None).  ``y``, ``final_state`` and ``workspace`` (uint8, at least
    workspace_bytes(...)) may be passed in to avoid allocation.  ``zoh``
    selects the exact zero-order-hold input weight (ssd_forward_zoh); ``z``
    [batch, L, H, P] (x's dtype) gates the output, y * silu(z)
    (ssd_forward_gated; not with ``zoh``).
    """
    lib = load()
    x = _dev(x, "x")
    dev = x.device
    code = _dtype_code(x)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _dev(dt, "dt", torch.float32, (batch, L, H), dev)
    _dev(A, "A", torch.float32, (H,), dev)
    _dev(B, "B", x.dtype, (batch, L, G, N), dev)
    _dev(C, "C", x.dtype, (batch, L, G, N), dev)
    _dev(D, "D", torch.float32, (H,), dev)
    _dev(init_state, "init_state", torch.float32, (batch, H, P, N), dev)
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape, dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=dev)
    _dev(final_state, "final_state", torch.float32, (batch, H, P, N), dev)
    need = lib.ssd_forward_workspace_bytes(batch, L, H, P, N, G, chunk, code)
    if need == 0:
        raise SSDError("ssd_forward_workspace_bytes", 3)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, None, dev)
    if z is not None:
        if zoh:
            raise ValueError("the gated forward has no zero-order-hold variant")
        _dev(z, "z", x.dtype, x.shape, dev)
        st = lib.ssd_forward_gated(batch, L, H, P, N, G, chunk, code, _p(x), _p(dt), _p(A), _p(B),
                                   _p(C), _p(D), _p(init_state), _p(z), _p(y), _p(final_state),
                                   _p(workspace), workspace.numel(), _stream(dev))
        _check("ssd_forward_gated", st)
        return y, final_state
    fn = lib.ssd_forward_zoh if zoh else lib.ssd_forward
    st = fn(batch, L, H, P, N, G, chunk, code, _p(x), _p(dt), _p(A), _p(B), _p(C),
            _p(D), _p(init_state), _p(y), _p(final_state), _p(workspace),
            workspace.numel(), _stream(dev))
    _check("ssd_forward_zoh" if zoh else "ssd_forward", st)
    return y, final_state


def ssm_step(state, x_t, dt_t, A, B_t, C_t, D=None, *, y_t=None, zoh=False):
    """One decode step; ``state`` [batch, H, P, N] fp32 is updated in place.
    x_t [batch, H, P]; dt_t [batch, H] fp32; B_t, C_t [batch, G, N].
    ``zoh`` selects the exact zero-order-hold input weight (ssm_step_zoh).
    Returns y_t [batch, H, P] in x_t's dtype."""
    lib = load()
    state = _dev(state, "state", torch.float32)
    dev = state.device
    batch, H, P, N = state.shape
    code = _dtype_code(x_t)
    G = B_t.shape[1]
    _dev(x_t, "x_t", None, (batch, H, P), dev)
    _dev(dt_t, "dt_t", torch.float32, (batch, H), dev)
    _dev(A, "A", torch.float32, (H,), dev)
    _dev(B_t, "B_t", x_t.dtype, (batch, G, N), dev)
    _dev(C_t, "C_t", x_t.dtype, (batch, G, N), dev)
    _dev(D, "D", torch.float32, (H,), dev)
    if y_t is None:
        y_t = torch.empty_like(x_t)
    _dev(y_t, "y_t", x_t.dtype, (batch, H, P), dev)
    fn = lib.ssm_step_zoh if zoh else lib.ssm_step
    st = fn(batch, H, P, N, G, code, _p(state), _p(x_t), _p(dt_t), _p(A), _p(B_t),
            _p(C_t), _p(D), _p(y_t), _stream(dev))
    _check("ssm_step_zoh" if zoh else "ssm_step", st)
    return y_t


# ----------------------------------------------------------------- stages
def chunk_cumsum(dt, A, chunk, zoh=False):
    """(cs [batch, H, nc, Q], dtc [batch, H, nc, Q]) -- see ssd_chunk_cumsum
    (ssd_chunk_cumsum_zoh when ``zoh``)."""
    lib = load()
    dt = _dev(dt, "dt", torch.float32)
    batch, L, H = dt.shape
    _dev(A, "A", torch.float32, (H,), dt.device)
    nc = n_chunks(L, chunk)
    cs = torch.empty((batch, H, nc, chunk), dtype=torch.float32, device=dt.device)
    dtc = torch.empty_like(cs)
    fn = lib.ssd_chunk_cumsum_zoh if zoh else lib.ssd_chunk_cumsum
    _check("ssd_chunk_cumsum", fn(batch, L, H, chunk, _p(dt), _p(A), _p(cs), _p(dtc),
                                  _stream(dt.device)))
    return cs, dtc


def chunk_state(x, B, cs, dtc, chunk):
    """S [batch, H, nc, P, N] in x's dtype -- see ssd_chunk_state."""
    lib = load()
    x = _dev(x, "x")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc = n_chunks(L, chunk)
    _dev(B, "B", x.dtype, (batch, L, G, N), x.device)
    _dev(cs, "cs", torch.float32, (batch, H, nc, chunk), x.device)
    _dev(dtc, "dtc", torch.float32, (batch, H, nc, chunk), x.device)
    S = torch.empty((batch, H, nc, P, N), dtype=x.dtype, device=x.device)
    _check("ssd_chunk_state", lib.ssd_chunk_state(batch, L, H, P, N, G, chunk, _dtype_code(x),
                                                  _p(x), _p(B), _p(cs), _p(dtc), _p(S),
                                                  _stream(x.device)))
    return S


def chunk_cumsum_state(x, B, dt, A, chunk):
    """(cs, dtc, S) -- see ssd_chunk_cumsum_state (the forward's first launch)."""
    lib = load()
    x = _dev(x, "x")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc = n_chunks(L, chunk)
    _dev(B, "B", x.dtype, (batch, L, G, N), x.device)
    _dev(dt, "dt", torch.float32, (batch, L, H), x.device)
    _dev(A, "A", torch.float32, (H,), x.device)
    cs = torch.empty((batch, H, nc, chunk), dtype=torch.float32, device=x.device)
    dtc = torch.empty_like(cs)
    S = torch.empty((batch, H, nc, P, N), dtype=x.dtype, device=x.device)
    _check("ssd_chunk_cumsum_state",
           lib.ssd_chunk_cumsum_state(batch, L, H, P, N, G, chunk, _dtype_code(x), _p(x), _p(B),
                                      _p(dt), _p(A), _p(cs), _p(dtc), _p(S), _stream(x.device)))
    return cs, dtc, S


def state_passing(S, cs, seqlen, chunk, dtype, init_state=None, final_state=None):
    """(Hin [batch, H, nc, P, N] in ``dtype``, final [batch, H, P, N] fp32)
    from S in ``dtype``."""
    lib = load()
    S = _dev(S, "S", dtype)
    batch, H, nc, P, N = S.shape
    _dev(cs, "cs", torch.float32, (batch, H, nc, chunk), S.device)
    _dev(init_state, "init_state", torch.float32, (batch, H, P, N), S.device)
    Hin = torch.empty((batch, H, nc, P, N), dtype=dtype, device=S.device)
    if final_state is None:
        final_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=S.device)
    _dev(final_state, "final_state", torch.float32, (batch, H, P, N), S.device)
    code = DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32
    _check("ssd_state_passing", lib.ssd_state_passing(batch, seqlen, H, P, N, chunk, code, _p(S),
                                                      _p(cs), _p(init_state), _p(Hin),
                                                      _p(final_state), _stream(S.device)))
    return Hin, final_state


def state_passing_seg(S, cs, seqlen, chunk, dtype, nsegments, init_state=None, final_state=None,
                      workspace=None):
    """(Hin, final) as state_passing, by the two-level associative scan over
    ``nsegments`` segments of chunks -- see ssd_state_passing_seg (S in
    ``dtype``)."""
    lib = load()
    S = _dev(S, "S", dtype)
    batch, H, nc, P, N = S.shape
    _dev(cs, "cs", torch.float32, (batch, H, nc, chunk), S.device)
    _dev(init_state, "init_state", torch.float32, (batch, H, P, N), S.device)
    Hin = torch.empty((batch, H, nc, P, N), dtype=dtype, device=S.device)
    if final_state is None:
        final_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=S.device)
    _dev(final_state, "final_state", torch.float32, (batch, H, P, N), S.device)
    need = lib.ssd_state_passing_seg_workspace_bytes(batch, H, P, N, nsegments)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=S.device)
    _dev(workspace, "workspace", torch.uint8, None, S.device)
    code = DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32
    _check("ssd_state_passing_seg",
           lib.ssd_state_passing_seg(batch, seqlen, H, P, N, chunk, nsegments, code, _p(S), _p(cs),
                                     _p(init_state), _p(Hin), _p(final_state), _p(workspace),
                                     workspace.numel(), _stream(S.device)))
    return Hin, final_state


def state_scan(x, B, cs, dtc, chunk, init_state=None, final_state=None):
    """(Hin [batch, H, nc, P, N] in x's dtype, final [batch, H, P, N] fp32) --
    see ssd_state_scan (chunk state and state passing in one pass)."""
    lib = load()
    x = _dev(x, "x")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc = n_chunks(L, chunk)
    _dev(B, "B", x.dtype, (batch, L, G, N), x.device)
    _dev(cs, "cs", torch.float32, (batch, H, nc, chunk), x.device)
    _dev(dtc, "dtc", torch.float32, (batch, H, nc, chunk), x.device)
    _dev(init_state, "init_state", torch.float32, (batch, H, P, N), x.device)
    Hin = torch.empty((batch, H, nc, P, N), dtype=x.dtype, device=x.device)
    if final_state is None:
        final_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=x.device)
    _dev(final_state, "final_state", torch.float32, (batch, H, P, N), x.device)
    _check("ssd_state_scan", lib.ssd_state_scan(batch, L, H, P, N, G, chunk, _dtype_code(x), _p(x),
                                                _p(B), _p(cs), _p(dtc), _p(init_state), _p(Hin),
                                                _p(final_state), _stream(x.device)))
    return Hin, final_state


def chunk_scan(x, B, C, cs, dtc, Hin, D, chunk, y=None):
    """y [batch, L, H, P] in x's dtype -- see ssd_chunk_scan."""
    lib = load()
    x = _dev(x, "x")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc = n_chunks(L, chunk)
    _dev(B, "B", x.dtype, (batch, L, G, N), x.device)
    _dev(C, "C", x.dtype, (batch, L, G, N), x.device)
    _dev(cs, "cs", torch.float32, (batch, H, nc, chunk), x.device)
    _dev(dtc, "dtc", torch.float32, (batch, H, nc, chunk), x.device)
    _dev(Hin, "Hin", x.dtype, (batch, H, nc, P, N), x.device)
    _dev(D, "D", torch.float32, (H,), x.device)
    if y is None:
        y = torch.empty_like(x)
    _check("ssd_chunk_scan", lib.ssd_chunk_scan(batch, L, H, P, N, G, chunk, _dtype_code(x), _p(x),
                                                _p(B), _p(C), _p(cs), _p(dtc), _p(Hin), _p(D),
                                                _p(y), _stream(x.device)))
    return y


def forward_run_chunks(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype) -> int:
    """The run length ssd_forward uses (0: the per-chunk stages) -- see
    ssd_forward_run_chunks."""
    code = dtype if isinstance(dtype, int) else (DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_F32)
    return int(load().ssd_forward_run_chunks(batch, seqlen, nheads, headdim, dstate, ngroups, chunk,
                                             code))


def chunk_state_runs(x, B, dt, A, chunk, run_chunks):
    """(cs, dtc, T [batch, H, nc, P, N], lam [batch, H, nc], rdec [batch, H, nruns])
    -- see ssd_chunk_state_runs (chunk states over runs of ``run_chunks``)."""
    lib = load()
    x = _dev(x, "x")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc = n_chunks(L, chunk)
    nruns = -(-nc // run_chunks)
    _dev(B, "B", x.dtype, (batch, L, G, N), x.device)
    _dev(dt, "dt", torch.float32, (batch, L, H), x.device)
    _dev(A, "A", torch.float32, (H,), x.device)
    cs = torch.empty((batch, H, nc, chunk), dtype=torch.float32, device=x.device)
    dtc = torch.empty_like(cs)
    T = torch.empty((batch, H, nc, P, N), dtype=x.dtype, device=x.device)
    lam = torch.empty((batch, H, nc), dtype=torch.float32, device=x.device)
    rdec = torch.empty((batch, H, nruns), dtype=torch.float32, device=x.device)
    _check("ssd_chunk_state_runs",
           lib.ssd_chunk_state_runs(batch, L, H, P, N, G, chunk, _dtype_code(x), run_chunks, _p(x),
                                    _p(B), _p(dt), _p(A), _p(cs), _p(dtc), _p(T), _p(lam), _p(rdec),
                                    _stream(x.device)))
    return cs, dtc, T, lam, rdec


def run_passing(T, rdec, seqlen, chunk, run_chunks, init_state=None, final_state=None):
    """(Hr [batch, H, nruns, P, N] in T's dtype, final [batch, H, P, N] fp32)
    -- see ssd_run_passing (the chain over runs)."""
    lib = load()
    T = _dev(T, "T")
    batch, H, nc, P, N = T.shape
    nruns = -(-nc // run_chunks)
    _dev(rdec, "rdec", torch.float32, (batch, H, nruns), T.device)
    _dev(init_state, "init_state", torch.float32, (batch, H, P, N), T.device)
    Hr = torch.empty((batch, H, nruns, P, N), dtype=T.dtype, device=T.device)
    if final_state is None:
        final_state = torch.empty((batch, H, P, N), dtype=torch.float32, device=T.device)
    _dev(final_state, "final_state", torch.float32, (batch, H, P, N), T.device)
    _check("ssd_run_passing",
           lib.ssd_run_passing(batch, seqlen, H, P, N, chunk, _dtype_code(T), run_chunks, _p(T),
                               _p(rdec), _p(init_state), _p(Hr), _p(final_state), _stream(T.device)))
    return Hr, final_state


def chunk_scan_runs(x, B, C, cs, dtc, T, Hr, lam, D, chunk, run_chunks, y=None):
    """y [batch, L, H, P] in x's dtype -- see ssd_chunk_scan_runs (each chunk's
    entering state formed from T and Hr)."""
    lib = load()
    x = _dev(x, "x")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc = n_chunks(L, chunk)
    nruns = -(-nc // run_chunks)
    _dev(B, "B", x.dtype, (batch, L, G, N), x.device)
    _dev(C, "C", x.dtype, (batch, L, G, N), x.device)
    _dev(cs, "cs", torch.float32, (batch, H, nc, chunk), x.device)
    _dev(dtc, "dtc", torch.float32, (batch, H, nc, chunk), x.device)
    _dev(T, "T", x.dtype, (batch, H, nc, P, N), x.device)
    _dev(Hr, "Hr", x.dtype, (batch, H, nruns, P, N), x.device)
    _dev(lam, "lam", torch.float32, (batch, H, nc), x.device)
    _dev(D, "D", torch.float32, (H,), x.device)
    if y is None:
        y = torch.empty_like(x)
    _check("ssd_chunk_scan_runs",
           lib.ssd_chunk_scan_runs(batch, L, H, P, N, G, chunk, _dtype_code(x), run_chunks, _p(x),
                                   _p(B), _p(C), _p(cs), _p(dtc), _p(T), _p(Hr), _p(lam), _p(D),
                                   _p(y), _stream(x.device)))
    return y


# ------------------------------------------------------ block around the scan
def layer_in(xbc, conv_w, conv_b, dt_raw, dt_bias, nheads, headdim, ngroups, dstate, *,
             x=None, B=None, C=None, dt=None):
    """The scan's inputs from a block's pre-activations -- see ssd_layer_in.

    xbc [batch, L, H*P + 2*G*N] (bf16 | fp32); conv_w [channels, K] fp32;
    conv_b [channels] fp32 or None; dt_raw [batch, L, H] fp32; dt_bias [H]
    fp32 or None.  Returns (x [batch, L, H, P], B [batch, L, G, N],
    C [batch, L, G, N] in xbc's dtype, dt [batch, L, H] fp32)."""
    lib = load()
    xbc = _dev(xbc, "xbc")
    dev = xbc.device
    batch, L, Cd = xbc.shape
    H, P, G, N = int(nheads), int(headdim), int(ngroups), int(dstate)
    if Cd != H * P + 2 * G * N:
        raise ValueError(f"xbc has {Cd} channels, expected H*P + 2*G*N = {H * P + 2 * G * N}")
    K = conv_w.shape[1] if conv_w.dim() == 2 else -1
    _dev(conv_w, "conv_w", torch.float32, (Cd, K), dev)
    _dev(conv_b, "conv_b", torch.float32, (Cd,), dev)
    _dev(dt_raw, "dt_raw", torch.float32, (batch, L, H), dev)
    _dev(dt_bias, "dt_bias", torch.float32, (H,), dev)
    if x is None:
        x = torch.empty((batch, L, H, P), dtype=xbc.dtype, device=dev)
    if B is None:
        B = torch.empty((batch, L, G, N), dtype=xbc.dtype, device=dev)
    if C is None:
        C = torch.empty((batch, L, G, N), dtype=xbc.dtype, device=dev)
    if dt is None:
        dt = torch.empty((batch, L, H), dtype=torch.float32, device=dev)
    _dev(x, "x", xbc.dtype, (batch, L, H, P), dev)
    _dev(B, "B", xbc.dtype, (batch, L, G, N), dev)
    _dev(C, "C", xbc.dtype, (batch, L, G, N), dev)
    _dev(dt, "dt", torch.float32, (batch, L, H), dev)
    _check("ssd_layer_in", lib.ssd_layer_in(batch, L, H, P, N, G, K, _dtype_code(xbc), _p(xbc),
                                            _p(conv_w), _p(conv_b), _p(dt_raw), _p(dt_bias),
                                            _p(x), _p(B), _p(C), _p(dt), _stream(dev)))
    return x, B, C, dt


def layer_out(y, z, out=None):
    """out = y * silu(z), elementwise (``out`` may be ``y``) -- see ssd_layer_out."""
    lib = load()
    y = _dev(y, "y")
    _dev(z, "z", y.dtype, y.shape, y.device)
    if out is None:
        out = torch.empty_like(y)
    _dev(out, "out", y.dtype, y.shape, y.device)
    _check("ssd_layer_out", lib.ssd_layer_out(y.numel(), _dtype_code(y), _p(y), _p(z), _p(out),
                                              _stream(y.device)))
    return out


def ssd_layer(xbc, z, dt_raw, A, D, conv_w, conv_b, dt_bias, nheads, headdim, ngroups, dstate,
              chunk=256, init_state=None, zoh=False):
    """The block around the scan, each step in the library's kernels:
    layer_in -> ssd_forward_gated (the gate inside the chunk scan's store where
    that applies), or ssd_forward_zoh -> layer_out for ``zoh``.  z [batch, L,
    H, P] in xbc's dtype.  Returns (out [batch, L, H, P], final_state [batch,
    H, P, N] fp32)."""
    x, B, C, dt = layer_in(xbc, conv_w, conv_b, dt_raw, dt_bias, nheads, headdim, ngroups, dstate)
    if zoh:
        y, fin = ssd_forward(x, dt, A, B, C, D, chunk, init_state, zoh=True)
        return layer_out(y, z, out=y), fin
    return ssd_forward(x, dt, A, B, C, D, chunk, init_state, z=z)
