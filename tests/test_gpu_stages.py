"""Each GPU stage against the fp64 stage definitions of oracle/stages.py,
feeding every stage the GPU's own upstream intermediates so that a mismatch
names one kernel.  Shapes span several chunks and a ragged last chunk."""
import math

import numpy as np
import pytest
import torch

from tests.helpers import TOL, say, to_gpu
from tests.metrics import max_rel_err

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


def _inputs(seed, batch, L, H, P, N, G, dtype, init=True):
    from mamba_ssd_scan_02_amd.workloads import ForwardSpec, make_forward_inputs
    spec = ForwardSpec("stage", batch, L, H, P, N, G, 64, dtype, init_var=0.1 if init else 0.0,
                       seed=seed)
    return make_forward_inputs(spec)


CASES = [
    # (name, batch, L, H, P, N, G, chunk, dtype)
    ("mfma_q256_ragged", 2, 700, 4, 64, 128, 2, 256, "bf16"),
    ("mfma_q128", 1, 512, 2, 64, 128, 1, 128, "bf16"),
    ("mfma_q64_ragged", 1, 333, 2, 64, 128, 2, 64, "bf16"),
    ("generic_f32", 2, 300, 3, 16, 16, 1, 64, "f32"),
    ("generic_f32_odd", 1, 77, 2, 3, 5, 1, 16, "f32"),
    ("generic_bf16", 1, 260, 2, 32, 64, 2, 128, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_stages(case):
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    name, batch, L, H, P, N, G, Q, dtype = case
    say(f"[stages] {name}")
    inp = _inputs(11, batch, L, H, P, N, G, dtype)
    g = to_gpu(inp)
    tol = TOL[dtype]

    # cumsum
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], Q)
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    err_cs = np.max(np.abs(cs.cpu().double().numpy() - Acs * LOG2E)) / max(1.0, np.abs(Acs * LOG2E).max())
    assert err_cs < 2e-6, err_cs
    nc = Acs.shape[2]
    dt_ref = np.zeros((batch, nc * Q, H), np.float32)
    dt_ref[:, :L] = inp["dt"].numpy()
    assert np.array_equal(dtc.cpu().numpy(), dt_ref.reshape(batch, nc, Q, H).transpose(0, 3, 1, 2))

    # chunk state, from the GPU's cs/dtc
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, Q)
    S_ref = stages.chunk_state(inp["x"], inp["dt"], inp["B"], Acs, Q)
    e = max_rel_err(S, S_ref)
    say(f"  chunk_state max rel err {e:.3e}")
    assert e < (tol if dtype == "bf16" else 1e-5)

    # state passing, from the GPU's S
    sd = torch.bfloat16 if dtype == "bf16" else torch.float32
    Hin, fin = ssd.state_passing(S, cs, L, Q, sd, g["init"])
    S_gpu = S.cpu().double().numpy()
    Hin_ref, fin_ref = stages.state_passing(S_gpu, Acs, inp["init"])
    e_h = max_rel_err(Hin, Hin_ref)
    e_f = max_rel_err(fin, fin_ref)
    say(f"  state_passing Hin {e_h:.3e} final {e_f:.3e}")
    assert e_h < (8e-3 if dtype == "bf16" else 1e-6)
    assert e_f < 1e-5

    # chunk scan, from the GPU's cs/dtc/Hin
    y = ssd.chunk_scan(g["x"], g["B"], g["C"], cs, dtc, Hin, g["D"], Q)
    y_ref = stages.chunk_scan(inp["x"], inp["dt"], inp["B"], inp["C"], Acs,
                              Hin.cpu().double().numpy(), inp["D"], Q)
    e_y = max_rel_err(y, y_ref)
    say(f"  chunk_scan max rel err {e_y:.3e}")
    assert e_y < tol


def test_chunk_scan_head_runs():
    """128 (batch, chunk, group) units of 25 heads: the launcher gives each
    workgroup a run of 13 or 12 heads of one chunk (on a 256-CU part), the
    path that keeps the C.B^T tiles in registers across a run.  The first and
    last head of both runs are checked against the oracle over every chunk,
    including the ragged last one."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    batch, L, H, P, N, G, Q = 1, 128 * 256 - 37, 25, 64, 128, 1, 256
    say("[stages] chunk_scan head runs")
    inp = _inputs(13, batch, L, H, P, N, G, "bf16")
    g = to_gpu(inp)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], Q)
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, Q)
    Hin, _ = ssd.state_passing(S, cs, L, Q, torch.bfloat16, g["init"])
    y = ssd.chunk_scan(g["x"], g["B"], g["C"], cs, dtc, Hin, g["D"], Q).cpu()
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    Hn = Hin.cpu().double().numpy()
    for h in (0, 12, 13, 24):
        sl = slice(h, h + 1)
        y_ref = stages.chunk_scan(inp["x"][:, :, sl], inp["dt"][:, :, sl], inp["B"], inp["C"],
                                  Acs[:, sl], Hn[:, sl], inp["D"][sl], Q)
        e = max_rel_err(y[:, :, sl], y_ref)
        say(f"  head {h}: max rel err {e:.3e}")
        assert e < TOL["bf16"], (h, e)


def test_chunk_scan_head_runs_strong_decay():
    """The head-run path with step sizes that make some 32-token tiles decay
    by far more than 2^64 (45-token windows at dt = 2.5 with A = -1, i.e.
    3.6 log2 units per token, between windows at dt = 0.05): those tiles,
    diagonal ones included, take the direct per-element weights and the
    rest the factorised ones.  First and last heads of both runs against the
    oracle over every chunk."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    batch, L, H, P, N, G, Q = 1, 128 * 256 - 37, 25, 64, 128, 1, 256
    say("[stages] chunk_scan head runs, strong decay")
    inp = _inputs(14, batch, L, H, P, N, G, "bf16")
    t = np.arange(L)
    win = np.where((t // 45) % 3 == 0, 2.5, 0.05).astype(np.float32)
    shift = np.arange(H) * 7                      # each head's windows start elsewhere
    dt = np.stack([np.roll(win, int(k)) for k in shift], axis=1)[None]
    inp["dt"] = torch.from_numpy(np.ascontiguousarray(dt))
    inp["A"] = torch.full((H,), -1.0, dtype=torch.float32)
    g = to_gpu(inp)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], Q)
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, Q)
    Hin, _ = ssd.state_passing(S, cs, L, Q, torch.bfloat16, g["init"])
    y = ssd.chunk_scan(g["x"], g["B"], g["C"], cs, dtc, Hin, g["D"], Q).cpu()
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    # both kinds of tile occur: some decay by more than 2^64, most by less
    tile_decay = (Acs[..., ::32] - Acs[..., 31::32]) * LOG2E
    assert (tile_decay > 64).any() and (tile_decay < 64).any()
    Hn = Hin.cpu().double().numpy()
    for h in (0, 12, 13, 24):
        sl = slice(h, h + 1)
        y_ref = stages.chunk_scan(inp["x"][:, :, sl], inp["dt"][:, :, sl], inp["B"], inp["C"],
                                  Acs[:, sl], Hn[:, sl], inp["D"][sl], Q)
        e = max_rel_err(y[:, :, sl], y_ref)
        say(f"  head {h}: max rel err {e:.3e}")
        assert e < TOL["bf16"], (h, e)


def test_stage_intermediates_deterministic():
    import mamba_ssd_scan_02_amd as ssd
    inp = _inputs(12, 1, 512, 4, 64, 128, 1, "bf16")
    g = to_gpu(inp)
    outs = []
    for _ in range(2):
        cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], 256)
        S = ssd.chunk_state(g["x"], g["B"], cs, dtc, 256)
        Hin, fin = ssd.state_passing(S, cs, 512, 256, torch.bfloat16, g["init"])
        y = ssd.chunk_scan(g["x"], g["B"], g["C"], cs, dtc, Hin, g["D"], 256)
        outs.append([t.clone() for t in (cs, S, Hin, fin, y)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


SCAN_CASES = [
    # (name, batch, L, H, G, init, alias init/final)
    ("one_chunk", 1, 256, 2, 1, True, False),
    ("ragged", 2, 700, 4, 2, True, False),
    ("one_token_tail", 1, 513, 3, 1, False, False),
    ("many_chunks", 1, 2600, 2, 2, True, False),
    ("short", 1, 40, 2, 1, True, False),
    ("aliased_state", 1, 600, 2, 1, True, True),
    ("head_pairs_two_groups", 2, 1000, 8, 2, True, False),
]


@pytest.mark.parametrize("case", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_state_scan(case):
    """The one-pass chunk-state + state-passing kernel against the fp64 stage
    definitions (Hin and final state), and against the two-kernel GPU path."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    name, batch, L, H, G, init, alias = case
    P, N, Q = 64, 128, 256
    say(f"[state_scan] {name}")
    inp = _inputs(21, batch, L, H, P, N, G, "bf16", init=init)
    g = to_gpu(inp)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], Q)
    st = g["init"].clone() if init else None
    fin_buf = st if alias else None
    Hin, fin = ssd.state_scan(g["x"], g["B"], cs, dtc, Q, init_state=st, final_state=fin_buf)
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    S_ref = stages.chunk_state(inp["x"], inp["dt"], inp["B"], Acs, Q)
    Hin_ref, fin_ref = stages.state_passing(S_ref, Acs, inp["init"] if init else None)
    e_h = max_rel_err(Hin, Hin_ref)
    e_f = max_rel_err(fin, fin_ref)
    say(f"  Hin {e_h:.3e} final {e_f:.3e}")
    assert e_h < TOL["bf16"] and e_f < TOL["bf16"]
    # the two-kernel path on the same device intermediates
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, Q)
    Hin2, fin2 = ssd.state_passing(S, cs, L, Q, torch.bfloat16, g["init"] if init else None)
    assert max_rel_err(Hin, Hin2.cpu().double().numpy()) < TOL["bf16"]
    assert max_rel_err(fin, fin2.cpu().double().numpy()) < TOL["bf16"]


def test_chunk_cumsum_zero_order_hold_weights():
    """ssd_chunk_cumsum_zoh: cs as the plain call, dtc = expm1(dt A) / A from
    the same fp32 inputs (fp64 on both sides, one rounding), dt where A = 0,
    0 past the end."""
    import mamba_ssd_scan_02_amd as ssd
    inp = _inputs(31, 2, 700, 5, 64, 128, 1, "bf16")
    inp["A"][2] = 0.0
    g = to_gpu(inp)
    cs0, _ = ssd.chunk_cumsum(g["dt"], g["A"], 256)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], 256, zoh=True)
    assert torch.equal(cs0, cs)
    dt = inp["dt"].numpy().astype(np.float64)
    A = inp["A"].numpy().astype(np.float64)
    w = np.where(A[None, None, :] == 0.0, dt, np.expm1(dt * A[None, None, :]) / np.where(A == 0.0, 1.0, A))
    nc = 3
    ref = np.zeros((2, nc * 256, 5))
    ref[:, :700] = w
    ref = ref.reshape(2, nc, 256, 5).transpose(0, 3, 1, 2).astype(np.float32)
    got = dtc.cpu().numpy()
    np.testing.assert_allclose(got, ref, rtol=2e-7, atol=0)
    assert np.array_equal(got[:, 2], ref[:, 2])   # A = 0: dt itself


SEG_CASES = [
    # (name, batch, L, H, P, N, Q, nsegments, dtype, init, alias init/final)
    ("one_segment", 2, 700, 3, 64, 128, 256, 1, "bf16", True, False),
    ("segment_per_chunk", 2, 700, 3, 64, 128, 256, 3, "bf16", True, False),
    ("more_segments_than_chunks", 1, 700, 2, 64, 128, 256, 9, "bf16", False, False),
    ("ragged_segments", 1, 65 * 64 + 17, 2, 64, 128, 64, 7, "bf16", True, False),
    ("many_segments", 1, 65 * 64 + 17, 2, 64, 128, 64, 33, "f32", True, True),
    ("scalar_lanes_f32", 2, 300, 2, 3, 5, 16, 4, "f32", True, False),
]


@pytest.mark.parametrize("case", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_state_passing_segmented(case):
    """ssd_state_passing_seg against the fp64 stage definition (from the GPU's
    own S and cs) and against the sequential GPU kernel."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    name, batch, L, H, P, N, Q, nseg, dtype, init, alias = case
    say(f"[state_passing_seg] {name}")
    inp = _inputs(41, batch, L, H, P, N, 1, dtype, init=init)
    g = to_gpu(inp)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], Q)
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, Q)
    sd = torch.bfloat16 if dtype == "bf16" else torch.float32
    st = g["init"].clone() if init else None
    Hin, fin = ssd.state_passing_seg(S, cs, L, Q, sd, nseg, init_state=st,
                                     final_state=st if alias else None)
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    Hin_ref, fin_ref = stages.state_passing(S.cpu().double().numpy(), Acs,
                                            inp["init"] if init else None)
    e_h, e_f = max_rel_err(Hin, Hin_ref), max_rel_err(fin, fin_ref)
    say(f"  Hin {e_h:.3e} final {e_f:.3e}")
    assert e_h < (8e-3 if dtype == "bf16" else 1e-6)
    assert e_f < 1e-5
    Hin2, fin2 = ssd.state_passing(S, cs, L, Q, sd, g["init"] if init else None)
    assert max_rel_err(fin, fin2.cpu().double().numpy()) < 1e-5
    assert max_rel_err(Hin, Hin2.cpu().double().numpy()) < (8e-3 if dtype == "bf16" else 1e-6)


def test_state_passing_segmented_errors():
    import mamba_ssd_scan_02_amd as ssd
    lib = ssd.load()
    t = torch.zeros(1 << 16, device="cuda")
    vp = t.data_ptr()
    need = lib.ssd_state_passing_seg_workspace_bytes(1, 2, 64, 128, 4)
    assert need > 0
    # workspace too small, NULL workspace, zero segments
    assert lib.ssd_state_passing_seg(1, 1024, 2, 64, 128, 256, 4, 1, vp, vp, None, vp, None, vp,
                                     need - 1, None) == 4
    assert lib.ssd_state_passing_seg(1, 1024, 2, 64, 128, 256, 4, 1, vp, vp, None, vp, None, None,
                                     need, None) == 4
    assert lib.ssd_state_passing_seg(1, 1024, 2, 64, 128, 256, 0, 1, vp, vp, None, vp, None, vp,
                                     need, None) == 2
    assert lib.ssd_state_passing_seg_workspace_bytes(1, 2, 64, 128, 0) == 0


def test_state_passing_segmented_long_context():
    """At the long-context shape (32 chains of 4,096 chunks) the segmented scan
    gives the sequential kernel's results up to rounding order (the
    sequential kernel is checked against the oracle by the 1M-token forward)."""
    import mamba_ssd_scan_02_amd as ssd
    from mamba_ssd_scan_02_amd.workloads import LONG_1M as spec
    say("[state_passing_seg] long context")
    b, L, H, P, N, Q = spec.batch, spec.seqlen, spec.nheads, spec.headdim, spec.dstate, spec.chunk
    nc = L // Q
    gen = torch.Generator(device="cuda").manual_seed(77)
    dt = torch.nn.functional.softplus(torch.randn(b, L, H, device="cuda", generator=gen) - 4.0)
    A = -torch.exp(torch.rand(H, device="cuda", generator=gen))
    cs, _ = ssd.chunk_cumsum(dt, A, Q)
    del dt
    S = torch.randn(b, H, nc, P, N, device="cuda", generator=gen) * 0.1
    init = torch.randn(b, H, P, N, device="cuda", generator=gen) * 0.3
    Hin, fin = ssd.state_passing(S, cs, L, Q, torch.bfloat16, init)
    Hin2, fin2 = ssd.state_passing_seg(S, cs, L, Q, torch.bfloat16, 64, init_state=init)
    e_f = ((fin2 - fin).abs().max() / fin.abs().max()).item()
    say(f"  final {e_f:.3e}")
    assert e_f < 1e-5
    # bf16 entering states: equal up to one rounding step
    d = (Hin2.float() - Hin.float()).abs()
    assert bool((d <= Hin.float().abs() * 2.0 ** -7 + 1e-6 * Hin.float().abs().max()).all())


def test_state_passing_segmented_deterministic():
    import mamba_ssd_scan_02_amd as ssd
    inp = _inputs(43, 2, 1000, 3, 64, 128, 1, "bf16")
    g = to_gpu(inp)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], 64)
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, 64)
    r1 = ssd.state_passing_seg(S, cs, 1000, 64, torch.bfloat16, 5, init_state=g["init"])
    r2 = ssd.state_passing_seg(S, cs, 1000, 64, torch.bfloat16, 5, init_state=g["init"])
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
