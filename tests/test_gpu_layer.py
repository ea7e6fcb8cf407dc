"""The block around the scan on the GPU (ssd_layer_in, ssd_layer_out and the
two composed with ssd_forward) against the fp64 definitions of
oracle/layer.py and the fp64 recurrence of the oracle.

Inputs: make_layer_inputs (seeded; see mamba_ssd_scan_02_amd/workloads.py).
Shapes cover the 8-channel vector path (H P and G N multiples of 8) and the
per-element path, filter widths 1..8, sequences shorter than the filter and
run lengths that leave ragged tails."""
import numpy as np
import pytest
import torch

from tests.helpers import TOL, say, to_gpu
from tests.metrics import gate, max_rel_err

pytestmark = pytest.mark.gpu

BF16_HALF_ULP = 2.0 ** -8     # |round_bf16(v) - v| <= 2^-8 |v| (8 significant bits)


def _spec(batch, L, H, P, N, G, dtype, chunk=256, init_var=0.0, seed=0):
    from mamba_ssd_scan_02_amd.workloads import ForwardSpec
    return ForwardSpec("layer", batch, L, H, P, N, G, chunk, dtype, init_var=init_var, seed=seed)


def _check_elem(got, ref, dtype):
    """bf16: within half a bf16 ulp of the fp64 value (plus fp32 arithmetic);
    f32: within 1e-5 of the tensor's largest magnitude."""
    g = got.detach().cpu().double().numpy()
    scale = float(np.max(np.abs(ref)))
    if dtype == "bf16":
        bound = BF16_HALF_ULP * (1 + 1e-5) * np.abs(ref) + 1e-6 * scale
    else:
        bound = 1e-5 * scale + 0 * ref
    bad = np.abs(g - ref) > bound
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:4].tolist())


LAYER_IN_CASES = [
    # (name, batch, L, H, P, N, G, K, dtype, biases)
    ("vec_bf16_k4_ragged", 2, 333, 4, 64, 128, 1, 4, "bf16", True),
    ("vec_f32_k2_groups", 1, 200, 4, 16, 16, 2, 2, "f32", True),
    ("vec_bf16_k8_shorter_than_filter", 2, 5, 2, 32, 64, 1, 8, "bf16", True),
    ("vec_bf16_k1", 1, 70, 2, 64, 128, 1, 1, "bf16", True),
    ("vec_f32_k3_no_bias", 1, 129, 2, 64, 128, 2, 3, "f32", False),
    ("vec_bf16_one_token", 3, 1, 2, 64, 128, 1, 4, "bf16", True),
    ("generic_f32_odd", 2, 77, 2, 3, 5, 1, 3, "f32", True),
    ("generic_bf16_odd_k7", 1, 130, 3, 5, 7, 1, 7, "bf16", False),
]


@pytest.mark.parametrize("case", LAYER_IN_CASES, ids=[c[0] for c in LAYER_IN_CASES])
def test_layer_in(case):
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import make_layer_inputs
    from oracle import layer

    name, batch, L, H, P, N, G, K, dtype, biases = case
    say(f"[layer_in] {name}")
    inp = make_layer_inputs(_spec(batch, L, H, P, N, G, dtype, seed=51), K)
    if not biases:
        inp["conv_b"] = None
        inp["dt_bias"] = None
    g = to_gpu(inp)
    x, B, C, dt = ssd.layer_in(g["xbc"], g["conv_w"], g["conv_b"], g["dt_raw"], g["dt_bias"],
                               H, P, G, N)
    torch.cuda.synchronize()
    xr, Br, Cr, dtr = layer.layer_in(inp["xbc"], inp["conv_w"], inp["conv_b"], inp["dt_raw"],
                                     inp["dt_bias"], H, P, G, N)
    for got, ref, nm in ((x, xr, "x"), (B, Br, "B"), (C, Cr, "C")):
        e = max_rel_err(got, ref)
        say(f"  {nm}: max rel err {e:.3e}")
        assert e < TOL[dtype], (nm, e)
        _check_elem(got, ref, dtype)
    e = max_rel_err(dt, dtr)
    say(f"  dt: max rel err {e:.3e}")
    assert e < 1e-5
    assert bool((dt > 0).all())


def test_layer_in_full_size_sampled():
    """The 2.7B-shaped layer (batch 4, 8192 tokens, 80 heads of 64, N = 128,
    K = 4) in one launch; the oracle checks the first tokens (zero padding),
    a window in the middle (with its K - 1 halo) and the last tokens of
    batch rows 0 and 3."""
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import make_layer_inputs
    from oracle import layer

    batch, L, H, P, N, G, K = 4, 8192, 80, 64, 128, 1, 4
    say("[layer_in] full size, sampled")
    inp = make_layer_inputs(_spec(batch, L, H, P, N, G, "bf16", seed=52), K)
    g = to_gpu(inp)
    x, B, C, dt = ssd.layer_in(g["xbc"], g["conv_w"], g["conv_b"], g["dt_raw"], g["dt_bias"],
                               H, P, G, N)
    torch.cuda.synchronize()
    for b in (0, 3):
        for t0, t1 in ((0, 200), (4000, 4130), (L - 150, L)):
            h0 = max(0, t0 - (K - 1))
            sl = slice(h0, t1)
            xr, Br, Cr, dtr = layer.layer_in(inp["xbc"][b:b + 1, sl], inp["conv_w"], inp["conv_b"],
                                             inp["dt_raw"][b:b + 1, sl], inp["dt_bias"], H, P, G, N)
            k = t0 - h0
            for got, ref in ((x, xr), (B, Br), (C, Cr)):
                gs = got[b:b + 1, t0:t1]
                assert max_rel_err(gs, ref[:, k:]) < TOL["bf16"]
                _check_elem(gs, ref[:, k:], "bf16")
            assert max_rel_err(dt[b:b + 1, t0:t1], dtr[:, k:]) < 1e-5


LAYER_OUT_CASES = [
    ("vec_bf16", (2, 300, 4, 64), "bf16", False),
    ("vec_f32_in_place", (1, 100, 2, 64), "f32", True),
    ("generic_f32_odd", (1, 77, 3, 5), "f32", False),
    ("generic_bf16_odd_in_place", (2, 31, 1, 3), "bf16", True),
]


@pytest.mark.parametrize("case", LAYER_OUT_CASES, ids=[c[0] for c in LAYER_OUT_CASES])
def test_layer_out(case):
    import mamba_ssd_scan_02_amd as ssd
    from oracle import layer

    name, shape, dtype, in_place = case
    say(f"[layer_out] {name}")
    sd = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(61)
    y = torch.randn(shape, generator=gen).to(sd)
    z = (torch.randn(shape, generator=gen) * 3).to(sd)
    ref = layer.layer_out(y, z)
    yg, zg = y.cuda(), z.cuda()
    out = ssd.layer_out(yg, zg, out=yg if in_place else None)
    torch.cuda.synchronize()
    if in_place:
        assert out.data_ptr() == yg.data_ptr()
    assert max_rel_err(out, ref) < TOL[dtype]
    _check_elem(out, ref, dtype)


def test_layer_errors():
    import mamba_ssd_scan_02_amd as ssd
    lib = ssd.load()
    t = torch.zeros(64, device="cuda")
    p = torch.zeros(64, device="cuda")
    vp = lambda a: a.data_ptr()
    # filter width outside 1..8
    assert lib.ssd_layer_in(1, 4, 1, 8, 8, 1, 9, 0, vp(t), vp(t), None, vp(t), None, vp(p),
                            vp(p), vp(p), vp(p), None) == 3
    # H % G != 0
    assert lib.ssd_layer_in(1, 4, 3, 8, 8, 2, 4, 0, vp(t), vp(t), None, vp(t), None, vp(p),
                            vp(p), vp(p), vp(p), None) == 2
    # a missing output
    assert lib.ssd_layer_in(1, 4, 1, 8, 8, 1, 4, 0, vp(t), vp(t), None, vp(t), None, None,
                            vp(p), vp(p), vp(p), None) == 1
    # the gate's output overlapping z
    assert lib.ssd_layer_out(16, 0, vp(t), vp(p), vp(p) + 4, None) == 7
    assert lib.ssd_layer_out(0, 0, vp(t), vp(p), vp(t), None) == 2


LAYER_CASES = [
    # (name, batch, L, H, P, N, G, K, chunk, dtype, init, zoh)
    ("bf16_ragged_init", 2, 700, 4, 64, 128, 1, 4, 256, "bf16", True, False),
    ("f32_generic", 1, 300, 2, 16, 16, 1, 4, 64, "f32", False, False),
    ("bf16_zoh_groups", 1, 520, 4, 64, 128, 2, 4, 256, "bf16", False, True),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_composed(case):
    """layer_in -> ssd_forward -> layer_out on the GPU against the fp64 layer
    steps around the oracle's recurrence.  The oracle's recurrence reads fp32
    inputs, so the fp64 layer_in outputs are rounded to fp32 once between the
    two (1e-7 relative, far below both tolerances)."""
    import oracle
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import make_layer_inputs
    from oracle import layer

    name, batch, L, H, P, N, G, K, Q, dtype, init, zoh = case
    say(f"[layer] {name}")
    inp = make_layer_inputs(_spec(batch, L, H, P, N, G, dtype, chunk=Q,
                                  init_var=0.1 if init else 0.0, seed=53), K)
    g = to_gpu(inp)
    out, fin = ssd.ssd_layer(g["xbc"], g["z"], g["dt_raw"], g["A"], g["D"], g["conv_w"],
                             g["conv_b"], g["dt_bias"], H, P, G, N, Q, g["init"], zoh=zoh)
    torch.cuda.synchronize()
    xr, Br, Cr, dtr = layer.layer_in(inp["xbc"], inp["conv_w"], inp["conv_b"], inp["dt_raw"],
                                     inp["dt_bias"], H, P, G, N)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    y_ref, fin_ref = oracle.forward_full(f32(xr), f32(dtr), inp["A"], f32(Br), f32(Cr),
                                         inp["D"], inp["init"], zoh=zoh)
    out_ref = layer.layer_out(y_ref, inp["z"])
    # magnitudes: the recurrence over absolute values of the same layer_in
    # outputs, through the gate's per-element factor |silu(z)|
    ab = lambda a: torch.from_numpy(np.ascontiguousarray(np.abs(a), dtype=np.float32))
    y_mag, fin_mag = oracle.forward_full(ab(xr), f32(dtr), inp["A"], ab(Br), ab(Cr),
                                         inp["D"].abs(), None if inp["init"] is None else
                                         inp["init"].abs(), zoh=zoh)
    out_mag = np.abs(layer.layer_out(y_mag, inp["z"]))
    gate(out, out_ref, TOL[dtype], "out", out_mag)
    gate(fin, fin_ref, TOL[dtype], "final_state", fin_mag)


def test_layer_bitwise_deterministic():
    """Two runs of the block's kernels on the same inputs give the same bits
    (no atomics, fixed reduction orders)."""
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import make_layer_inputs
    inp = make_layer_inputs(_spec(2, 333, 4, 64, 128, 2, "bf16", init_var=0.1, seed=54), 4)
    g = to_gpu(inp)
    outs = []
    for _ in range(2):
        out, fin = ssd.ssd_layer(g["xbc"], g["z"], g["dt_raw"], g["A"], g["D"], g["conv_w"],
                                 g["conv_b"], g["dt_bias"], 4, 64, 2, 128, 256, g["init"])
        outs.append((out.clone(), fin.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


GATED_CASES = [
    # (name, batch, L, H, P, N, G, chunk, dtype) -- the first three reach the
    # 256-token matrix-core chunk scan (the gate inside its store), the rest
    # the gate kernel after the scan
    ("resident_ragged_groups", 2, 700, 4, 64, 128, 2, 256, "bf16"),
    ("resident_130m_heads", 2, 1024, 24, 64, 128, 1, 256, "bf16"),
    ("resident_one_chunk", 1, 100, 2, 64, 128, 1, 256, "bf16"),
    ("short_q128", 1, 520, 2, 64, 128, 1, 128, "bf16"),
    ("short_q64", 1, 333, 2, 64, 128, 2, 64, "bf16"),
    ("generic_f32", 1, 300, 3, 16, 16, 1, 64, "f32"),
    # the two-level form (runs of K = 2 chunks; the gate in the same store)
    ("runs_two_level", 1, 32768, 32, 64, 128, 1, 256, "bf16"),
]


@pytest.mark.parametrize("case", GATED_CASES, ids=[c[0] for c in GATED_CASES])
def test_forward_gated_matches_forward_then_gate(case):
    """ssd_forward_gated gives, bit for bit, what ssd_forward followed by
    ssd_layer_out(y, z, out = y) gives, with its outputs and workspace
    guarded (canary bands, NaN fill); the final state is unchanged."""
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import make_forward_inputs
    from tests.helpers import Guarded

    name, batch, L, H, P, N, G, Q, dtype = case
    say(f"[gated] {name}")
    if name.startswith("runs"):
        assert ssd.forward_run_chunks(batch, L, H, P, N, G, Q, torch.bfloat16) > 0
    inp = make_forward_inputs(_spec(batch, L, H, P, N, G, dtype, chunk=Q, init_var=0.1, seed=61))
    g = to_gpu(inp)
    x = g["x"]
    gen = torch.Generator(device="cpu").manual_seed(62)
    z = torch.randn(x.shape, generator=gen, dtype=torch.float32).to(x.dtype).cuda()
    y_ref, f_ref = ssd.ssd_forward(x, g["dt"], g["A"], g["B"], g["C"], g["D"], Q, g["init"])
    out_ref = ssd.layer_out(y_ref, z, out=y_ref.clone())
    yb = Guarded(tuple(x.shape), x.dtype)
    fb = Guarded((batch, H, P, N), torch.float32)
    wb = Guarded((ssd.workspace_bytes(batch, L, H, P, N, G, Q, x.dtype),), torch.uint8)
    out, fin = ssd.ssd_forward(x, g["dt"], g["A"], g["B"], g["C"], g["D"], Q, g["init"], y=yb.t,
                               final_state=fb.t, workspace=wb.t, z=z)
    torch.cuda.synchronize()
    assert yb.intact() and fb.intact() and wb.intact(), "a store landed outside its array"
    assert torch.equal(out, out_ref), (name, max_rel_err(out, out_ref.cpu().double().numpy()))
    assert torch.equal(fin, f_ref)
