"""End-to-end parity of ssd_forward (GPU, through the C ABI) with the fp64
oracle, on the five workloads and on the edge cases the method has.

Gates (tests/metrics.py), per output tensor, at 1e-4 for fp32 storage and
2e-2 for bf16 storage (fp32 accumulation and state): max |gpu - oracle| /
max |oracle|, and max |gpu - oracle| / (|oracle| + rms(oracle)) per element.
At full size the oracle runs on a sample of (batch, head) pairs over the
whole sequence (first and last pair always included).  Every full-size
workload is also run without the skip term (D = None): with D ~ N(0, 1) the
D x term sets the output's peak, so only a D-free run gates the scan terms
(the masked in-chunk product and the carried state) at their own scale.
Outputs and the workspace are guarded and NaN-poisoned (tests/helpers.py)."""
import math

import numpy as np
import pytest
import torch

from tests.helpers import (TOL, abs_inputs, all_pairs, gpu_forward, oracle_forward,
                           oracle_forward_scaled, sample_pairs, say, select_state, select_y,
                           to_gpu)
from tests.metrics import gate, max_rel_err

pytestmark = pytest.mark.gpu


def _check(inp, chunk, dtype, bh=None, t_range=None, label=""):
    y, fin = gpu_forward(inp, chunk)
    batch, L, H, P = inp["x"].shape
    if bh is None:
        bh = all_pairs(batch, H)
    y_ref, f_ref, y_mag, f_mag = oracle_forward_scaled(inp, bh=bh, t_range=t_range)
    say(f"[forward] {label} chunk={chunk}")
    gate(select_y(y, bh, t_range), y_ref, TOL[dtype], "y", y_mag)
    gate(select_state(fin, bh), f_ref, TOL[dtype], "final_state", f_mag)
    return y, fin


def _check_with_and_without_skip(inp, chunk, dtype, bh=None, label=""):
    """The workload as drawn, then the same inputs with D = None."""
    _check(inp, chunk, dtype, bh=bh, label=label)
    _check(dict(inp, D=None), chunk, dtype, bh=bh, label=label + " D=None")


def _spec_inputs(spec):
    from mamba_ssd_scan_02_amd.workloads import make_forward_inputs
    return make_forward_inputs(spec)


# ----------------------------------------------------------------- workloads
def test_tiny_f32():
    from mamba_ssd_scan_02_amd.workloads import TINY_F32
    _check_with_and_without_skip(_spec_inputs(TINY_F32), TINY_F32.chunk, "f32",
                                 label=TINY_F32.name)


def test_mamba2_130m_shape():
    """130M-shaped layer: 24 heads per group, which chunk_scan's resident
    kernel takes in four runs of 6 heads per chunk."""
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M as s
    inp = _spec_inputs(s)
    _check_with_and_without_skip(inp, s.chunk, s.dtype,
                                 bh=sample_pairs(s.batch, s.nheads, 24, seed=2), label=s.name)


def test_mamba2_2p7b_shape():
    """2.7B-shaped layer (the bench workload): 80 heads per group, so
    chunk_scan runs the resident kernel (runs of 40 heads)."""
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_2P7B as s
    inp = _spec_inputs(s)
    _check_with_and_without_skip(inp, s.chunk, s.dtype,
                                 bh=sample_pairs(s.batch, s.nheads, 12, seed=3), label=s.name)


@pytest.mark.parametrize("chunk", [128, 64])
def test_mamba2_2p7b_shape_short_chunks(chunk):
    """The 2.7B-shaped layer cut into 128- or 64-token chunks (64 or 128 per
    sequence): the matrix-core kernels for short chunks, chunk_scan in runs
    of all 80 heads of a chunk."""
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_2P7B as s
    inp = _spec_inputs(s)
    _check_with_and_without_skip(inp, chunk, s.dtype,
                                 bh=sample_pairs(s.batch, s.nheads, 6, seed=4), label=s.name)


def test_long_context_1m():
    """One 1M-token sequence, 8 groups of 4 heads (resident chunk_scan in runs
    of a whole group, 4,096 chained chunks).  One head of every group, at
    every position within a group: heads 0, 5, 10, 15, 16, 21, 26 and 31."""
    from mamba_ssd_scan_02_amd.workloads import LONG_1M as s
    inp = _spec_inputs(s)
    say(f"[forward] {s.name}: inputs ready")
    _check_with_and_without_skip(inp, s.chunk, s.dtype,
                                 bh=[(0, h) for h in (0, 5, 10, 15, 16, 21, 26, 31)], label=s.name)


# ---------------------------------------------------------------- edge cases
def test_water_tank_in_tiny_shape():
    """Inflow 2 on channel 0 with half kept per step: 2, 3, 3.5, 3.75, 3.875,
    3.9375 on channel 0 and 0 everywhere else (page "State Space Model",
    section "Un sistema che riassume il passato")."""
    import mamba_ssd_scan_02_amd as ssd
    L, P, N = 6, 16, 16
    x = torch.zeros(1, L, 1, P)
    x[..., 0] = 2.0
    dt = torch.ones(1, L, 1)
    A = torch.tensor([-math.log(2.0)])
    B = torch.zeros(1, L, 1, N)
    B[..., 0] = 1.0
    y, fin = ssd.ssd_forward(x.cuda(), dt.cuda(), A.cuda(), B.cuda(), B.clone().cuda(), None, 64)
    y = y.cpu()
    np.testing.assert_allclose(y[0, :, 0, 0].numpy(), [2, 3, 3.5, 3.75, 3.875, 3.9375], atol=2e-6)
    assert torch.all(y[0, :, 0, 1:] == 0)
    # resume: half of 3.875 plus two new litres
    init = torch.zeros(1, 1, P, N)
    init[0, 0, 0, 0] = 3.875
    y2, _ = ssd.ssd_forward(x[:, :1].cuda(), dt[:, :1].cuda(), A.cuda(), B[:, :1].cuda(),
                            B[:, :1].clone().cuda(), None, 64, init.cuda())
    assert abs(float(y2[0, 0, 0, 0]) - 3.9375) < 2e-6


def test_long_memory_bf16():
    """Tiny |A|: chunks barely decay, so every carried state matters."""
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M
    inp = _spec_inputs(MAMBA2_130M.with_(batch=2, seqlen=2048, nheads=8, init_var=0.1))
    r = np.random.default_rng(5)
    inp["A"] = torch.from_numpy((-1e-4 * np.exp(r.uniform(0, 1, 8))).astype(np.float32))
    _check(inp, 256, "bf16", label="long_memory")


def test_long_memory_f32():
    from mamba_ssd_scan_02_amd.workloads import TINY_F32
    inp = _spec_inputs(TINY_F32.with_(batch=2, seqlen=1000, nheads=3, init_var=0.5))
    inp["A"] = torch.tensor([-1e-3, -1e-4, -1e-2], dtype=torch.float32)
    _check(inp, 64, "f32", label="long_memory_f32")


@pytest.mark.parametrize("chunk", [256, 128, 64])
@pytest.mark.parametrize("L", [1, 63, 255, 257, 1000])
def test_ragged_lengths_bf16(L, chunk):
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M
    inp = _spec_inputs(MAMBA2_130M.with_(batch=2, seqlen=L, nheads=4, init_var=0.1, seed=77))
    _check_with_and_without_skip(inp, chunk, "bf16", label=f"ragged L={L}")


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_chunk_sweep_bf16(chunk):
    """Same inputs, three chunk sizes: all match the oracle."""
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M
    inp = _spec_inputs(MAMBA2_130M.with_(batch=2, seqlen=1024, nheads=4, init_var=0.1, seed=78))
    _check_with_and_without_skip(inp, chunk, "bf16", label="chunk sweep")


@pytest.mark.parametrize("chunk", [1, 7, 64, 200, 256])
def test_chunk_sweep_f32(chunk):
    from mamba_ssd_scan_02_amd.workloads import TINY_F32
    inp = _spec_inputs(TINY_F32.with_(batch=2, seqlen=300, nheads=2, init_var=0.3, seed=79))
    _check(inp, chunk, "f32", label="chunk sweep f32")


@pytest.mark.parametrize("chunk", [256, 128, 64])
def test_groups_and_permutation(chunk):
    """G = 8 groups of 4 heads; permuting groups together with their heads
    permutes the outputs exactly."""
    from mamba_ssd_scan_02_amd.workloads import LONG_1M
    inp = _spec_inputs(LONG_1M.with_(seqlen=1024, init_var=0.1, seed=80))
    y, fin = _check(inp, chunk, "bf16", label="groups G=8")
    gperm = np.array([3, 0, 7, 1, 6, 2, 5, 4])
    hperm = np.concatenate([np.arange(4 * g, 4 * g + 4) for g in gperm])
    p = dict(inp)
    p["B"], p["C"] = inp["B"][:, :, gperm].contiguous(), inp["C"][:, :, gperm].contiguous()
    p["x"], p["dt"] = inp["x"][:, :, hperm].contiguous(), inp["dt"][:, :, hperm].contiguous()
    p["A"], p["D"] = inp["A"][hperm].contiguous(), inp["D"][hperm].contiguous()
    p["init"] = inp["init"][:, hperm].contiguous()
    y2, fin2 = gpu_forward(p, chunk)
    assert torch.equal(y2.cpu(), y.cpu()[:, :, hperm])
    assert torch.equal(fin2.cpu(), fin.cpu()[:, hperm])


def test_split_sequence_handoff():
    """forward(x[:m]) then forward(x[m:], init=final) equals forward(x): the
    single-device form of carrying boundary states between sequence shards."""
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M
    inp = _spec_inputs(MAMBA2_130M.with_(batch=2, seqlen=1536, nheads=4, init_var=0.1, seed=81))
    m = 512 + 100
    first = {k: (v[:, :m].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    second = {k: (v[:, m:].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    y1, f1 = gpu_forward(first, 256)
    second["init"] = f1.cpu()
    y2, f2 = gpu_forward(second, 256)
    y_ref, f_ref, y_mag, f_mag = oracle_forward_scaled(inp)
    bh = all_pairs(2, 4)
    y_cat = torch.cat([y1.cpu(), y2.cpu()], dim=1)
    say("[forward] handoff")
    gate(select_y(y_cat, bh), y_ref, TOL["bf16"], "y", y_mag)
    gate(select_state(f2, bh), f_ref, TOL["bf16"], "final_state", f_mag)


def test_zero_step_keeps_state():
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M
    inp = _spec_inputs(MAMBA2_130M.with_(batch=1, seqlen=300, nheads=2, init_var=0.1, seed=82))
    inp["dt"] = torch.zeros_like(inp["dt"])
    y, fin = _check(inp, 256, "bf16", label="dt=0")
    assert torch.equal(fin.cpu(), inp["init"])


def test_huge_step_is_memoryless():
    from mamba_ssd_scan_02_amd.workloads import TINY_F32
    inp = _spec_inputs(TINY_F32.with_(batch=1, seqlen=128, nheads=2, init_var=0.3, seed=83))
    inp["dt"] = torch.full_like(inp["dt"], 50.0)
    _check(inp, 64, "f32", label="dt=50")


def test_no_skip_no_init_no_final():
    """D = None, init = None, final_state not requested."""
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M
    inp = _spec_inputs(MAMBA2_130M.with_(batch=1, seqlen=512, nheads=2, seed=84))
    g = to_gpu(inp)
    y, fin = ssd.ssd_forward(g["x"], g["dt"], g["A"], g["B"], g["C"], None, 256, None,
                             return_final_state=False)
    assert fin is None
    ref = dict(inp, D=None, init=None)
    y_ref, _, y_mag, _ = oracle_forward_scaled(ref)
    gate(select_y(y, all_pairs(1, 2)), y_ref, TOL["bf16"], "y (no D, no init)", y_mag)


def test_final_state_may_alias_init():
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M
    inp = _spec_inputs(MAMBA2_130M.with_(batch=1, seqlen=512, nheads=2, init_var=0.1, seed=85))
    g = to_gpu(inp)
    y_a, f_a = ssd.ssd_forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 256, g["init"])
    st = g["init"].clone()
    y_b, f_b = ssd.ssd_forward(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 256, st,
                               final_state=st)
    assert torch.equal(y_a, y_b) and torch.equal(f_a, st)


def test_final_state_may_alias_init_two_level():
    """The same on the two-level path (32 heads, 128 chunks: runs of two
    chunks), where only the chain over runs reads the initial state and
    writes the final one; inputs drawn on the device."""
    import mamba_ssd_scan_02_amd as ssd
    batch, L, H, P, N, G, Q = 1, 32768, 32, 64, 128, 1, 256
    assert ssd.forward_run_chunks(batch, L, H, P, N, G, Q, torch.bfloat16) > 0
    gen = torch.Generator(device="cuda").manual_seed(86)
    rn = lambda *sh: torch.randn(*sh, generator=gen, device="cuda")
    x = rn(batch, L, H, P).to(torch.bfloat16)
    dt = torch.nn.functional.softplus(rn(batch, L, H) - 2.0)
    A = -torch.exp(torch.rand(H, generator=gen, device="cuda") * 1.5)
    Bm = (rn(batch, L, G, N) / N ** 0.5).to(torch.bfloat16)
    Cm = (rn(batch, L, G, N) / N ** 0.5).to(torch.bfloat16)
    D = rn(H)
    init = rn(batch, H, P, N) * 0.3
    y_a, f_a = ssd.ssd_forward(x, dt, A, Bm, Cm, D, Q, init)
    st = init.clone()
    y_b, f_b = ssd.ssd_forward(x, dt, A, Bm, Cm, D, Q, st, final_state=st)
    assert torch.equal(y_a, y_b) and torch.equal(f_a, st)


def test_bitwise_deterministic():
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M
    inp = _spec_inputs(MAMBA2_130M.with_(batch=2, seqlen=1024, nheads=8, init_var=0.1, seed=86))
    y1, f1 = gpu_forward(inp, 256)
    y2, f2 = gpu_forward(inp, 256)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


# ------------------------------------------------- exact zero-order hold (f4)
@pytest.mark.parametrize("case", [
    # (label, spec changes, chunk, sampled pairs)
    ("bf16_2p7b_shape", dict(), 256, 12),
    ("bf16_130m_ragged", dict(batch=2, seqlen=1500), 256, None),
    ("f32_generic", dict(batch=2, seqlen=300, nheads=3, headdim=16, dstate=16, dtype="f32"), 64, None),
])
def test_zero_order_hold_forward(case):
    """ssd_forward_zoh against the oracle's zero-order-hold recurrence, with
    steps long enough (dt ~ softplus(z + 1)) that the hold's weight
    expm1(dt A) / A is far from dt; the plain forward must then differ."""
    from mamba_ssd_scan_02_amd.workloads import MAMBA2_130M, MAMBA2_2P7B
    label, changes, chunk, nsample = case
    base = MAMBA2_2P7B if label.startswith("bf16_2p7b") else MAMBA2_130M
    spec = base.with_(dt_shift=1.0, **changes)
    inp = _spec_inputs(spec)
    batch, L, H, P = inp["x"].shape
    bh = all_pairs(batch, H) if nsample is None else sample_pairs(batch, H, nsample, seed=9)
    y, fin = gpu_forward(inp, chunk, zoh=True)
    y_ref, f_ref, y_mag, f_mag = oracle_forward_scaled(inp, bh=bh, zoh=True)
    say(f"[forward zoh] {label}")
    gate(select_y(y, bh), y_ref, TOL[spec.dtype], "y", y_mag)
    gate(select_state(fin, bh), f_ref, TOL[spec.dtype], "final_state", f_mag)
    y_plain, _ = gpu_forward(inp, chunk)
    d = max_rel_err(select_y(y_plain, bh), y_ref)
    assert d > 10 * TOL[spec.dtype], d


CONV_CASES = [
    # (label, batch, L, H, P, N, G, chunk, dtype, zoh)
    ("bf16_mfma", 2, 700, 4, 64, 128, 2, 256, "bf16", False),
    ("bf16_mfma_zoh", 1, 600, 2, 64, 128, 1, 128, "bf16", True),
    ("f32_generic", 1, 333, 3, 16, 32, 1, 64, "f32", False),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_time_invariant_is_a_convolution(case):
    """With dt, B and C constant over the tokens (the time-invariant case of
    page "State Space Model", section "Un sistema che riassume il passato"),
    the GPU forward equals the causal convolution of x with the kernel
    K_k = (C . B) w a^k (a = exp(dt A), w = dt or expm1(dt A) / A), D x added,
    computed here by FFT from the same stored values -- no recurrence."""
    from scipy.signal import fftconvolve

    label, batch, L, H, P, N, G, chunk, dtype, zoh = case
    say(f"[forward conv] {label}")
    sd = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(77)
    x = torch.from_numpy(rng.standard_normal((batch, L, H, P)).astype(np.float32)).to(sd)
    dt_h = np.log1p(np.exp(rng.standard_normal((batch, H)) - 1.0)).astype(np.float32)
    A = (-np.exp(rng.uniform(0.0, 1.0, H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    Bv = torch.from_numpy((rng.standard_normal((batch, G, N)) / math.sqrt(N)).astype(np.float32)).to(sd)
    Cv = torch.from_numpy((rng.standard_normal((batch, G, N)) / math.sqrt(N)).astype(np.float32)).to(sd)
    dt = torch.from_numpy(np.repeat(dt_h[:, None, :], L, axis=1))
    B = Bv[:, None].expand(batch, L, G, N).contiguous()
    C = Cv[:, None].expand(batch, L, G, N).contiguous()
    inp = dict(x=x, dt=dt, A=torch.from_numpy(A), B=B, C=C, D=torch.from_numpy(D), init=None)
    y, _ = gpu_forward(inp, chunk, zoh=zoh)

    x64 = x.double().numpy()
    B64, C64 = Bv.double().numpy(), Cv.double().numpy()
    ref = np.empty_like(x64)
    mag = np.empty_like(x64)      # the same convolution over absolute values
    k = np.arange(L, dtype=np.float64)
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            d, a_h = float(dt_h[b, h]), float(A[h])
            w = math.expm1(d * a_h) / a_h if zoh else d
            K = float(C64[b, g] @ B64[b, g]) * w * np.exp(d * a_h * k)
            Km = float(np.abs(C64[b, g]) @ np.abs(B64[b, g])) * abs(w) * np.exp(d * a_h * k)
            ref[b, :, h] = fftconvolve(x64[b, :, h], K[:, None], axes=0)[:L] + float(D[h]) * x64[b, :, h]
            mag[b, :, h] = (np.abs(fftconvolve(np.abs(x64[b, :, h]), Km[:, None], axes=0)[:L]) +
                            abs(float(D[h])) * np.abs(x64[b, :, h]))
    gate(y, ref, TOL[dtype], "y", mag)
