"""Each GPU stage against the fp64 stage definitions of oracle/stages.py,
feeding every stage the GPU's own upstream intermediates so that a mismatch
names one kernel.  Shapes span several chunks and a ragged last chunk."""
import math

import numpy as np
import pytest
import torch

from tests.helpers import TOL, say, to_gpu
from tests.metrics import gate, max_rel_err

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
    ("mfma_q128_groups_ragged", 2, 1000, 6, 64, 128, 3, 128, "bf16"),
    ("mfma_q64_ragged", 1, 333, 2, 64, 128, 2, 64, "bf16"),
    ("mfma_q64_odd_heads", 2, 700, 6, 64, 128, 2, 64, "bf16"),
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
    S_mag = stages.chunk_state(inp["x"].abs(), inp["dt"], inp["B"].abs(), Acs, Q)
    gate(S, S_ref, tol if dtype == "bf16" else 1e-5, "chunk_state S", S_mag)

    # the forward's first launch (the cumsum inside the chunk-state kernel
    # where that applies) gives the same cs, dtc and S, bit for bit
    cs2, dtc2, S2 = ssd.chunk_cumsum_state(g["x"], g["B"], g["dt"], g["A"], Q)
    assert torch.equal(cs2, cs) and torch.equal(dtc2, dtc), "cs / dtc of the fused launch"
    assert torch.equal(S2, S), "S of the fused launch"

    # state passing, from the GPU's S
    sd = torch.bfloat16 if dtype == "bf16" else torch.float32
    Hin, fin = ssd.state_passing(S, cs, L, Q, sd, g["init"])
    S_gpu = S.cpu().double().numpy()
    Hin_ref, fin_ref = stages.state_passing(S_gpu, Acs, inp["init"])
    Hin_mag, fin_mag = stages.state_passing(np.abs(S_gpu), Acs, inp["init"].abs())
    gate(Hin, Hin_ref, 8e-3 if dtype == "bf16" else 1e-6, "state_passing Hin", Hin_mag)
    gate(fin, fin_ref, 1e-5, "state_passing final", fin_mag)

    # chunk scan, from the GPU's cs/dtc/Hin, with and without the skip term
    Hn = Hin.cpu().double().numpy()
    for D_gpu, D_ref, what in ((g["D"], inp["D"], "chunk_scan y"),
                               (None, None, "chunk_scan y (D=None)")):
        y = ssd.chunk_scan(g["x"], g["B"], g["C"], cs, dtc, Hin, D_gpu, Q)
        y_ref = stages.chunk_scan(inp["x"], inp["dt"], inp["B"], inp["C"], Acs, Hn, D_ref, Q)
        y_mag = stages.chunk_scan(inp["x"].abs(), inp["dt"], inp["B"].abs(), inp["C"].abs(), Acs,
                                  np.abs(Hn), None if D_ref is None else D_ref.abs(), Q)
        gate(y, y_ref, tol, what, y_mag)


def test_chunk_state_many_rounds():
    """800 head-pair workgroups (100 chunks x 8 pairs), more than one round of
    the machine (three per CU), each storing its S tiles through LDS as whole
    rows: S and the forward's first launch against the fp64 stage
    definition."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    batch, L, H, P, N, G, Q = 1, 256 * 100 - 3, 16, 64, 128, 2, 256
    say("[stages] chunk_state, many rounds")
    inp = _inputs(15, batch, L, H, P, N, G, "bf16")
    g = to_gpu(inp)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], Q)
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, Q)
    cs2, dtc2, S2 = ssd.chunk_cumsum_state(g["x"], g["B"], g["dt"], g["A"], Q)
    assert torch.equal(cs2, cs) and torch.equal(dtc2, dtc) and torch.equal(S2, S)
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    S_ref = stages.chunk_state(inp["x"], inp["dt"], inp["B"], Acs, Q)
    S_mag = stages.chunk_state(inp["x"].abs(), inp["dt"], inp["B"].abs(), Acs, Q)
    gate(S, S_ref, TOL["bf16"], "chunk_state S (many rounds)", S_mag)


@pytest.mark.parametrize("Q", [256, 128, 64])
@pytest.mark.parametrize("skip", [True, False], ids=["with_D", "D_none"])
def test_chunk_scan_head_runs(skip, Q):
    """25 heads over 32,731 tokens: with 256-token chunks (128 (batch, chunk,
    group) units) the launcher gives each workgroup a run of 13 or 12 heads
    of one chunk (on a 256-CU part), with 128- and 64-token chunks (256 and
    512 units) one run of all 25 -- the paths that keep the C.B^T tiles in
    registers across a run.  Heads 0, 12, 13 and 24 are checked against the oracle over every
    chunk, including the ragged last one; with D = None the masked in-chunk
    product and the carried state are gated at their own scale."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    batch, L, H, P, N, G = 1, 128 * 256 - 37, 25, 64, 128, 1
    say(f"[stages] chunk_scan head runs, chunk {Q} ({'with D' if skip else 'D=None'})")
    inp = _inputs(13, batch, L, H, P, N, G, "bf16")
    g = to_gpu(inp)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], Q)
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, Q)
    Hin, _ = ssd.state_passing(S, cs, L, Q, torch.bfloat16, g["init"])
    y = ssd.chunk_scan(g["x"], g["B"], g["C"], cs, dtc, Hin, g["D"] if skip else None, Q).cpu()
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    Hn = Hin.cpu().double().numpy()
    for h in (0, 12, 13, 24):
        sl = slice(h, h + 1)
        y_ref = stages.chunk_scan(inp["x"][:, :, sl], inp["dt"][:, :, sl], inp["B"], inp["C"],
                                  Acs[:, sl], Hn[:, sl], inp["D"][sl] if skip else None, Q)
        y_mag = stages.chunk_scan(inp["x"][:, :, sl].abs(), inp["dt"][:, :, sl], inp["B"].abs(),
                                  inp["C"].abs(), Acs[:, sl], np.abs(Hn[:, sl]),
                                  inp["D"][sl].abs() if skip else None, Q)
        gate(y[:, :, sl], y_ref, TOL["bf16"], f"head {h}", y_mag)


@pytest.mark.parametrize("skip", [True, False], ids=["with_D", "D_none"])
def test_chunk_scan_head_runs_strong_decay(skip):
    """The head-run path with step sizes that make some 32-token tiles decay
    by far more than 2^64 (45-token windows at dt = 2.5 with A = -1, i.e.
    3.6 log2 units per token, between windows at dt = 0.05): those tiles,
    diagonal ones included, take the direct per-element weights and the
    rest the factorised ones.  First and last heads of both runs against the
    oracle over every chunk."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    batch, L, H, P, N, G, Q = 1, 128 * 256 - 37, 25, 64, 128, 1, 256
    say(f"[stages] chunk_scan head runs, strong decay ({'with D' if skip else 'D=None'})")
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
    y = ssd.chunk_scan(g["x"], g["B"], g["C"], cs, dtc, Hin, g["D"] if skip else None, Q).cpu()
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    # both kinds of tile occur: some decay by more than 2^64, most by less
    tile_decay = (Acs[..., ::32] - Acs[..., 31::32]) * LOG2E
    assert (tile_decay > 64).any() and (tile_decay < 64).any()
    Hn = Hin.cpu().double().numpy()
    for h in (0, 12, 13, 24):
        sl = slice(h, h + 1)
        y_ref = stages.chunk_scan(inp["x"][:, :, sl], inp["dt"][:, :, sl], inp["B"], inp["C"],
                                  Acs[:, sl], Hn[:, sl], inp["D"][sl] if skip else None, Q)
        y_mag = stages.chunk_scan(inp["x"][:, :, sl].abs(), inp["dt"][:, :, sl], inp["B"].abs(),
                                  inp["C"].abs(), Acs[:, sl], np.abs(Hn[:, sl]),
                                  inp["D"][sl].abs() if skip else None, Q)
        gate(y[:, :, sl], y_ref, TOL["bf16"], f"head {h}", y_mag)


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
    # (name, batch, L, H, G, chunk, init, alias init/final); an even head
    # count per group takes the walked (head-pair) kernel, an odd one the
    # per-head kernel
    ("one_chunk", 1, 256, 2, 1, 256, True, False),
    ("ragged", 2, 700, 4, 2, 256, True, False),
    ("one_token_tail", 1, 513, 3, 1, 256, False, False),
    ("many_chunks", 1, 2600, 2, 2, 256, True, False),
    ("short", 1, 40, 2, 1, 256, True, False),
    ("aliased_state", 1, 600, 2, 1, 256, True, True),
    ("head_pairs_two_groups", 2, 1000, 8, 2, 256, True, False),
    ("walk_many_chunks", 1, 40 * 256 + 77, 4, 1, 256, True, False),
    ("walk_chunk128_ragged", 2, 1000, 4, 1, 128, True, False),
    ("walk_chunk128_one_chunk", 1, 100, 2, 1, 128, False, False),
    ("walk_chunk128_aliased", 1, 33 * 128, 6, 3, 128, True, True),
]


@pytest.mark.parametrize("case", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_state_scan(case):
    """The one-pass chunk-state + state-passing kernels against the fp64
    stage definitions (Hin and final state), and against the two-kernel GPU
    path."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    name, batch, L, H, G, Q, init, alias = case
    P, N = 64, 128
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
    S_mag = stages.chunk_state(inp["x"].abs(), inp["dt"], inp["B"].abs(), Acs, Q)
    Hin_mag, fin_mag = stages.state_passing(S_mag, Acs, inp["init"].abs() if init else None)
    gate(Hin, Hin_ref, TOL["bf16"], "Hin", Hin_mag)
    gate(fin, fin_ref, TOL["bf16"], "final", fin_mag)
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
    S_gpu = S.cpu().double().numpy()
    Hin_ref, fin_ref = stages.state_passing(S_gpu, Acs, inp["init"] if init else None)
    Hin_mag, fin_mag = stages.state_passing(np.abs(S_gpu), Acs,
                                            inp["init"].abs() if init else None)
    gate(Hin, Hin_ref, 8e-3 if dtype == "bf16" else 1e-6, "Hin", Hin_mag)
    gate(fin, fin_ref, 1e-5, "final", fin_mag)
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
    gives the sequential kernel's results up to rounding order, and both
    match the fp64 stage definition on a sample of heads and state entries
    over the whole chain."""
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
    S = (torch.randn(b, H, nc, P, N, device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    init = torch.randn(b, H, P, N, device="cuda", generator=gen) * 0.3
    Hin, fin = ssd.state_passing(S, cs, L, Q, torch.bfloat16, init)
    Hin2, fin2 = ssd.state_passing_seg(S, cs, L, Q, torch.bfloat16, 64, init_state=init)
    e_f = ((fin2 - fin).abs().max() / fin.abs().max()).item()
    say(f"  final {e_f:.3e}")
    assert e_f < 1e-5
    # bf16 entering states: equal up to one rounding step
    d = (Hin2.float() - Hin.float()).abs()
    assert bool((d <= Hin.float().abs() * 2.0 ** -7 + 1e-6 * Hin.float().abs().max()).all())

    # both kernels against the fp64 stage definition on a sample: two heads,
    # 256 of the 8,192 state entries, every one of the 4,096 chunks (from the
    # GPU's S and the host's fp64 prefix of dt A)
    from oracle import stages
    heads = [0, H - 1]
    idx = torch.from_numpy(np.random.default_rng(78).choice(P * N, 256, replace=False)).cuda()
    sub = lambda t: t[0, heads].reshape(len(heads), nc, P * N)[:, :, idx]          # [2, nc, 256]
    S_sub = sub(S).cpu().double().numpy()[None, :, :, None, :]                   # [1, 2, nc, 1, 256]
    init_sub = init[0, heads].reshape(len(heads), P * N)[:, idx].cpu().double().numpy()[None, :, None, :]
    gen = torch.Generator(device="cuda").manual_seed(77)
    dt = torch.nn.functional.softplus(torch.randn(b, L, H, device="cuda", generator=gen) - 4.0)
    A_h = A.cpu().double().numpy()
    dt_h = dt[:, :, heads].cpu().double().numpy()
    del dt
    Acs = stages.chunk_cumsum(dt_h, A_h[heads], Q)                               # [1, 2, nc, Q]
    Hin_ref, fin_ref = stages.state_passing(S_sub, Acs, init_sub)
    Hin_mag, fin_mag = stages.state_passing(np.abs(S_sub), Acs, np.abs(init_sub))
    for what, Hx, fx in (("sequential", Hin, fin), ("segmented", Hin2, fin2)):
        Hs = sub(Hx).float()[None, :, :, None, :]
        fs = fx[0, heads].reshape(len(heads), P * N)[:, idx][None, :, None, :]
        gate(Hs, Hin_ref, 8e-3, f"{what} Hin (sampled)", Hin_mag)
        gate(fs, fin_ref, 1e-5, f"{what} final (sampled)", fin_mag)


def test_state_passing_segmented_deterministic():
    import mamba_ssd_scan_02_amd as ssd
    inp = _inputs(43, 2, 1000, 3, 64, 128, 1, "bf16")
    g = to_gpu(inp)
    cs, dtc = ssd.chunk_cumsum(g["dt"], g["A"], 64)
    S = ssd.chunk_state(g["x"], g["B"], cs, dtc, 64)
    r1 = ssd.state_passing_seg(S, cs, 1000, 64, torch.bfloat16, 5, init_state=g["init"])
    r2 = ssd.state_passing_seg(S, cs, 1000, 64, torch.bfloat16, 5, init_state=g["init"])
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])



RUN_CASES = [
    # (name, batch, L, H, G, run length K)
    ("runs_k3_ragged_groups", 2, 256 * 9 - 37, 4, 2, 3),
    ("runs_k4_exact", 1, 256 * 8, 2, 1, 4),
    ("runs_k1", 1, 256 * 3 - 5, 2, 1, 1),
    ("runs_k16_one_run", 2, 256 * 5, 4, 1, 16),
]


@pytest.mark.parametrize("case", RUN_CASES, ids=[c[0] for c in RUN_CASES])
def test_two_level_stages(case):
    """The two-level recurrence between chunks, stage by stage against the
    fp64 definitions, each stage fed the GPU's own upstream outputs: chunk
    states over runs of K chunks (T, lam, rdec, and the cumsum rows bit for
    bit those of the forward's per-chunk first launch), the chain over runs
    (Hr, final), and the chunk scan forming each chunk's entering state from
    T and Hr (with and without the skip term)."""
    import mamba_ssd_scan_02_amd as ssd
    from oracle import stages

    name, batch, L, H, G, K = case
    P, N, Q = 64, 128, 256
    say(f"[stages] {name}")
    inp = _inputs(23, batch, L, H, P, N, G, "bf16")
    g = to_gpu(inp)
    tol = TOL["bf16"]
    LN2 = math.log(2.0)

    cs, dtc, T, lam, rdec = ssd.chunk_state_runs(g["x"], g["B"], g["dt"], g["A"], Q, K)
    cs1, dtc1, S1 = ssd.chunk_cumsum_state(g["x"], g["B"], g["dt"], g["A"], Q)
    assert torch.equal(cs, cs1) and torch.equal(dtc, dtc1), "cumsum rows of the run walk"
    Acs = stages.chunk_cumsum(inp["dt"], inp["A"], Q)
    S_ref = stages.chunk_state(inp["x"], inp["dt"], inp["B"], Acs, Q)
    S_mag = stages.chunk_state(inp["x"].abs(), inp["dt"], inp["B"].abs(), Acs, Q)
    T_ref, lam_ref, rdec_ref = stages.run_states(S_ref, Acs, K)
    T_mag, _, _ = stages.run_states(S_mag, Acs, K)
    gate(T, T_ref, tol, "chunk_state_runs T", T_mag)
    scale = max(1.0, float(np.abs(rdec_ref).max()))
    err_lam = np.max(np.abs(lam.cpu().double().numpy() * LN2 - lam_ref)) / scale
    err_rdec = np.max(np.abs(rdec.cpu().double().numpy() * LN2 - rdec_ref)) / scale
    say(f"  lam {err_lam:.2e}  rdec {err_rdec:.2e}")
    assert err_lam < 2e-6 and err_rdec < 2e-6, (err_lam, err_rdec)

    # the chain over runs, from the GPU's T and rdec
    Hr, fin = ssd.run_passing(T, rdec, L, Q, K, g["init"])
    T_gpu = T.cpu().double().numpy()
    rdec_gpu = rdec.cpu().double().numpy() * LN2
    Hr_ref, fin_ref = stages.run_passing(T_gpu, rdec_gpu, K, inp["init"])
    Hr_mag, fin_mag = stages.run_passing(np.abs(T_gpu), rdec_gpu, K, inp["init"].abs())
    gate(Hr, Hr_ref, 8e-3, "run_passing Hr", Hr_mag)
    gate(fin, fin_ref, 1e-5, "run_passing final", fin_mag)

    # the final state against the per-chunk chain on the fp64 S
    _, fin_chain = stages.state_passing(S_ref, Acs, inp["init"])
    _, fin_chain_mag = stages.state_passing(S_mag, Acs, inp["init"].abs())
    gate(fin, fin_chain, tol, "run_passing final vs the per-chunk chain", fin_chain_mag)

    # chunk scan from the GPU's T, Hr and lam: each entering state is formed
    # (and rounded once to bf16) in the kernel
    Hin = stages.runs_entering_states(T_gpu, Hr.cpu().double().numpy(),
                                      lam.cpu().double().numpy() * LN2, K)
    Hin_mag = stages.runs_entering_states(np.abs(T_gpu), np.abs(Hr.cpu().double().numpy()),
                                          lam.cpu().double().numpy() * LN2, K)
    for D_gpu, D_ref, what in ((g["D"], inp["D"], "chunk_scan_runs y"),
                               (None, None, "chunk_scan_runs y (D=None)")):
        y = ssd.chunk_scan_runs(g["x"], g["B"], g["C"], cs, dtc, T, Hr, lam, D_gpu, Q, K)
        y_ref = stages.chunk_scan(inp["x"], inp["dt"], inp["B"], inp["C"], Acs, Hin, D_ref, Q)
        y_mag = stages.chunk_scan(inp["x"].abs(), inp["dt"], inp["B"].abs(), inp["C"].abs(), Acs,
                                  Hin_mag, None if D_ref is None else D_ref.abs(), Q)
        gate(y, y_ref, tol, what, y_mag)
