"""ssm_step (GPU, through the C ABI) against the oracle's step, one token at a
time: y_t at every step and the state at steps 1, 2, 4, ..., 64, both gates of
tests/metrics.py.  The state and every y_t sit inside canary guard bands
(y_t NaN-filled before each step), checked after every step."""
import math

import numpy as np
import pytest
import torch

from tests.helpers import TOL, Guarded, say, to_gpu
from tests.metrics import gate, max_rel_err

pytestmark = pytest.mark.gpu


def _run_decode(spec, check_every_state=False, zoh=False):
    import mamba_ssd_scan_02_amd as ssd
    import oracle
    from mamba_ssd_scan_02_amd.workloads import make_decode_static, make_decode_step
    st = make_decode_static(spec)
    sg = Guarded(tuple(st["state"].shape), torch.float32, fill=None)
    sg.t.copy_(st["state"].cuda())
    state_gpu = sg.t
    state_ref = st["state"].double().numpy().copy()
    state_mag = np.abs(state_ref)        # the same steps over absolute values
    A, D = st["A"].cuda(), st["D"].cuda()
    worst_y = worst_s = 0.0
    say(f"[decode] {spec.name}")
    for t in range(spec.steps):
        s = make_decode_step(spec, t)
        g = to_gpu(s)
        yg = Guarded(tuple(g["x"].shape), g["x"].dtype)
        y = ssd.ssm_step(state_gpu, g["x"], g["dt"], A, g["B"], g["C"], D, y_t=yg.t, zoh=zoh)
        torch.cuda.synchronize()
        assert yg.intact() and sg.intact(), f"a store landed outside y_t or the state at step {t}"
        y_ref = oracle.step(state_ref, s["x"], s["dt"], st["A"], s["B"], s["C"], st["D"], zoh=zoh)
        y_mag = oracle.step(state_mag, s["x"].abs(), s["dt"], st["A"], s["B"].abs(), s["C"].abs(),
                            st["D"].abs(), zoh=zoh)
        e_y = max(gate(y, y_ref, TOL[spec.dtype], f"step {t} y_t", y_mag))
        worst_y = max(worst_y, e_y)
        k = t + 1
        if check_every_state or (k & (k - 1)) == 0 or k == spec.steps:
            e_s = max(gate(state_gpu, state_ref, TOL[spec.dtype], f"step {t} state", state_mag))
            worst_s = max(worst_s, e_s)
    say(f"[decode] {spec.name}: worst y {worst_y:.3e} worst state {worst_s:.3e}")


def test_decode_b256_64_steps():
    from mamba_ssd_scan_02_amd.workloads import DECODE_B256
    _run_decode(DECODE_B256)


def test_decode_small_shapes():
    from mamba_ssd_scan_02_amd.workloads import DECODE_B256
    for kw in (dict(batch=3, nheads=4, headdim=64, dstate=128, ngroups=2, steps=9),
               dict(batch=2, nheads=3, headdim=16, dstate=16, ngroups=1, steps=5, dtype="f32"),
               dict(batch=2, nheads=2, headdim=5, dstate=7, ngroups=1, steps=5, dtype="f32"),
               dict(batch=1, nheads=2, headdim=32, dstate=256, ngroups=2, steps=4),
               dict(batch=1, nheads=1, headdim=1, dstate=1, ngroups=1, steps=3, dtype="f32")):
        _run_decode(DECODE_B256.with_(name=f"decode {kw}", **kw), check_every_state=True)


def test_decode_water_tank():
    import mamba_ssd_scan_02_amd as ssd
    state = torch.zeros(1, 1, 1, 4, device="cuda")
    x = torch.full((1, 1, 1), 2.0, device="cuda")
    dt = torch.ones(1, 1, device="cuda")
    A = torch.tensor([-math.log(2.0)], device="cuda")
    Bv = torch.tensor([[[1.0, 0, 0, 0]]], device="cuda")
    got = [float(ssd.ssm_step(state, x, dt, A, Bv, Bv.clone())[0, 0, 0]) for _ in range(6)]
    np.testing.assert_allclose(got, [2, 3, 3.5, 3.75, 3.875, 3.9375], atol=2e-6)


def test_prefill_then_decode():
    """forward over L tokens, then ssm_step for k more tokens, equals the
    oracle over L + k tokens."""
    import mamba_ssd_scan_02_amd as ssd
    import oracle
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M, make_forward_inputs
    L, k = 700, 6
    inp = make_forward_inputs(MAMBA2_130M.with_(batch=2, seqlen=L + k, nheads=4, init_var=0.1,
                                                seed=90))
    g = to_gpu(inp)
    y, fin = ssd.ssd_forward(g["x"][:, :L].contiguous(), g["dt"][:, :L].contiguous(), g["A"],
                             g["B"][:, :L].contiguous(), g["C"][:, :L].contiguous(), g["D"], 256,
                             g["init"])
    y_ref, f_ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                  inp["init"])
    state = fin
    for t in range(L, L + k):
        yt = ssd.ssm_step(state, g["x"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"],
                          g["B"][:, t].contiguous(), g["C"][:, t].contiguous(), g["D"])
        ref = y_ref.reshape(2, 4, L + k, 64)[:, :, t]
        gate(yt, ref, TOL["bf16"], f"decode token {t}")
    gate(state, f_ref.reshape(2, 4, 64, 128), TOL["bf16"], "state after decode")


def test_decode_zero_order_hold():
    """ssm_step_zoh (input weight expm1(dt A) / A) against the oracle's step with
    the same discretisation, on the vector kernel (N = 128) and the generic one
    (N = 20), with steps large enough that the two discretisations differ."""
    from mamba_ssd_scan_02_amd.workloads import DECODE_B256
    for spec in (DECODE_B256.with_(batch=4, steps=12, dt_shift=1.0, a_hi=2.0, name="zoh_n128"),
                 DECODE_B256.with_(batch=3, steps=9, nheads=6, ngroups=2, headdim=7, dstate=20,
                                   dtype="f32", dt_shift=1.0, a_hi=2.0, name="zoh_n20_f32")):
        _run_decode(spec, check_every_state=True, zoh=True)
