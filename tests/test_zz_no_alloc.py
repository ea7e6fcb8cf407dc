"""ssd_forward_noalloc -- ssd_forward with its workspace in the library's
per-device scratch array, for callers that cannot allocate -- called through
the C ABI and checked against ssd_forward on the same inputs (bitwise: the
same kernels run) and against the oracle (the parity gates), on two calls in
a row, the second with a smaller input, so that the second call runs over
whatever the first left in the array."""
import ctypes

import pytest
import torch

from tests.helpers import TOL, Guarded, all_pairs, oracle_forward_scaled, sample_pairs, say
from tests.helpers import select_state, select_y, to_gpu
from tests.metrics import gate

pytestmark = pytest.mark.gpu


def _noalloc(lib, g, chunk):
    x = g["x"]
    batch, L, H, P = x.shape
    G, N = g["B"].shape[2], g["B"].shape[3]
    yb = Guarded(tuple(x.shape), x.dtype)
    fb = Guarded((batch, H, P, N), torch.float32)
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = 1 if x.dtype == torch.bfloat16 else 0
    st = lib.ssd_forward_noalloc(batch, L, H, P, N, G, chunk, code, p(x), p(g["dt"]), p(g["A"]),
                                 p(g["B"]), p(g["C"]), p(g.get("D")), p(g.get("init")), p(yb.t),
                                 p(fb.t), stream)
    assert st == 0, st
    torch.cuda.synchronize()
    assert yb.intact() and fb.intact()
    return yb.t, fb.t


def test_noalloc_matches_forward_on_two_calls():
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M, make_forward_inputs
    lib = ssd.load()
    cases = [
        # the 130M-shaped layer (53 MB of workspace), then a smaller, ragged one
        ("mamba2_130m", MAMBA2_130M, sample_pairs(8, 24, 12, seed=21)),
        ("ragged_small", MAMBA2_130M.with_(batch=2, seqlen=700, nheads=4, ngroups=2,
                                           init_var=0.1, seed=22), all_pairs(2, 4)),
    ]
    for name, spec, bh in cases:
        say(f"[noalloc] {name}")
        inp = make_forward_inputs(spec)
        g = to_gpu(inp)
        y, fin = _noalloc(lib, g, spec.chunk)
        y_ref, f_ref = ssd.ssd_forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], spec.chunk,
                                       g["init"])
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(fin, f_ref)
        yo, fo, ym, fm = oracle_forward_scaled(inp, bh=bh)
        gate(select_y(y, bh), yo, TOL[spec.dtype], "y", ym)
        gate(select_state(fin, bh), fo, TOL[spec.dtype], "final_state", fm)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """The 2.7B-shaped layer needs more workspace than the array holds: the
    call returns SSD_ERR_WORKSPACE before any launch."""
    import mamba_ssd_scan_02_amd as ssd
    lib = ssd.load()
    t = torch.zeros(1 << 10, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    assert lib.ssd_forward_workspace_bytes(4, 8192, 80, 64, 128, 1, 256, 1) > 64 << 20
    assert lib.ssd_forward_noalloc(4, 8192, 80, 64, 128, 1, 256, 1, p, p, p, p, p, None, None, p,
                                   None, None) == 4
