"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test states what fixes the expected value: numbers printed on the pages
(tests/golden/), a closed form, a brute-force construction of a different
shape (materialised matrix, convolution sum, masked matmul), an invariant, or
a limit.  Together they fail on the plausible mistakes: a dropped D or init
term, a read-out before the update, a wrong sign of the decay, a transposed or
swapped B/C, a wrong head->group map, a wrong chunk boundary.
"""
import json
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_case(seed, batch=2, L=40, H=4, P=3, N=5, G=2, with_init=True, with_D=True,
               a_scale=1.0, dt_scale=1.0):
    r = _rng(seed)
    x = r.standard_normal((batch, L, H, P)).astype(np.float32)
    dt = (np.log1p(np.exp(r.standard_normal((batch, L, H)) - 1.0)) * dt_scale).astype(np.float32)
    A = (-np.exp(r.uniform(0, 1, H)) * a_scale).astype(np.float32)
    B = (r.standard_normal((batch, L, G, N)) / math.sqrt(N)).astype(np.float32)
    C = (r.standard_normal((batch, L, G, N)) / math.sqrt(N)).astype(np.float32)
    D = r.standard_normal(H).astype(np.float32) if with_D else None
    init = r.standard_normal((batch, H, P, N)).astype(np.float32) if with_init else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, init=init)


def _tank_inputs(L, x_val=2.0, init=None):
    """One head, one channel, one state entry: inflow x, half kept each step
    (dt = 1, A = -ln 2 so exp(dt A) = 1/2), B = C = 1, no skip term."""
    x = np.full((1, L, 1, 1), x_val, dtype=np.float32)
    dt = np.ones((1, L, 1), dtype=np.float32)
    A = np.array([-math.log(2.0)], dtype=np.float32)
    one = np.ones((1, L, 1, 1), dtype=np.float32)
    init_a = None if init is None else np.full((1, 1, 1, 1), init, dtype=np.float32)
    return x, dt, A, one, one, init_a


# --------------------------------------------------------------------------
# Page "State Space Model", section "Un sistema che riassume il passato":
# the water-tank worked example.
# --------------------------------------------------------------------------
def test_water_tank_levels(oracle_mod):
    g = json.loads((GOLDEN / "water_tank.json").read_text())
    levels = g["levels_read_each_minute_from_empty"]
    assert g["first_level_is_the_empty_tank"] and levels[0] == 0
    expected = levels[1:] + [g["level_after_3_875"]]
    x, dt, A, B, C, _ = _tank_inputs(len(expected))
    # A is stored in fp32, so the kept fraction is exp(fp32(-ln 2)) = 1/2 up
    # to 3e-8; the levels below agree with the page to that accuracy.
    y, fin = oracle_mod.forward(x, dt, A, B, C)
    np.testing.assert_allclose(y[0, :, 0], expected, rtol=0, atol=1e-6)
    assert fin[0, 0, 0] == pytest.approx(y[0, -1, 0], abs=0)


def test_water_tank_exact_kept_fraction_in_fractions():
    """The page's sequence is the recurrence level <- level/2 + 2 from 0, which
    in exact rationals gives 2, 3, 7/2, 15/4, 31/8, 63/16 and tends to 4."""
    g = json.loads((GOLDEN / "water_tank.json").read_text())
    lvl = Fraction(0)
    seq = []
    for _ in range(6):
        lvl = lvl * Fraction(1, 2) + 2
        seq.append(lvl)
    assert [float(v) for v in seq[:5]] == g["levels_read_each_minute_from_empty"][1:]
    assert float(seq[5]) == g["level_after_3_875"]
    assert 4 - seq[5] == Fraction(1, 16) and g["settles_at"] == 4


def test_water_tank_settles_at_four(oracle_mod):
    x, dt, A, B, C, _ = _tank_inputs(80)
    y, _ = oracle_mod.forward(x, dt, A, B, C)
    assert y[0, -1, 0] == pytest.approx(4.0, abs=1e-5)
    d1 = np.diff(y[0, :, 0])
    assert np.all(d1[:20] > 0) and np.all(d1 >= 0)   # rises, ever more slowly
    assert np.all(d1[1:20] < d1[:19])


def test_water_tank_filter_weights_and_fading(oracle_mod):
    """A single pour at t = 0 fades by half a minute: weights 1, 1/2, 1/4, ...;
    1/32 is left after five minutes and less than 1e-9 after thirty."""
    g = json.loads((GOLDEN / "water_tank.json").read_text())
    L = 31
    x, dt, A, B, C, _ = _tank_inputs(L, x_val=0.0)
    x[0, 0, 0, 0] = 1.0
    y, _ = oracle_mod.forward(x, dt, A, B, C)
    w = y[0, :, 0]
    np.testing.assert_allclose(w[:4], g["fading_weights_now_1_2_3_minutes_ago"], atol=1e-7)
    assert w[5] == pytest.approx(g["fraction_left_of_a_pour_after_5_minutes"], rel=1e-6)
    assert 0 < w[30] < g["fraction_left_of_a_pour_after_30_minutes_is_below"]
    # the filter view: 3.875 is the sum of the first five weights times 2
    assert 2 * w[:5].sum() == pytest.approx(3.875, abs=1e-6)
    # one minute later the filter covers six pours: the oldest, faded five
    # times, adds 2 * 1/32 = 0.0625 and the sum reaches 3.9375
    assert 2 * w[5] == pytest.approx(g["weight_added_for_the_sixth_pour"], abs=1e-7)
    assert 2 * w[:6].sum() == pytest.approx(g["level_after_3_875"], abs=1e-6)


def test_water_tank_resume_from_3_875(oracle_mod):
    """Half of 3.875 plus the two new litres is 3.9375: the state handed in as
    the initial state is decayed once and then receives the new input."""
    g = json.loads((GOLDEN / "water_tank.json").read_text())
    x, dt, A, B, C, init = _tank_inputs(1, init=3.875)
    y, fin = oracle_mod.forward(x, dt, A, B, C, init=init)
    assert y[0, 0, 0] == pytest.approx(g["level_after_3_875"], abs=1e-6)
    st = init.astype(np.float64).copy()
    yt = oracle_mod.step(st, x[:, 0], dt[:, 0], A, B[:, 0], C[:, 0])
    assert yt[0, 0, 0] == pytest.approx(g["level_after_3_875"], abs=1e-6)
    assert st[0, 0, 0, 0] == pytest.approx(fin[0, 0, 0], abs=0)


def test_water_tank_inside_a_wide_head(oracle_mod):
    """The tank on channel 0 / state entry 0 of a P = N = 16 head, all other
    entries idle: channel 0 reproduces the tank, every other output is 0."""
    L, P, N = 6, 16, 16
    x = np.zeros((1, L, 1, P), np.float32)
    x[..., 0] = 2.0
    dt = np.ones((1, L, 1), np.float32)
    A = np.array([-math.log(2.0)], np.float32)
    B = np.zeros((1, L, 1, N), np.float32)
    B[..., 0] = 1.0
    C = B.copy()
    y, _ = oracle_mod.forward(x, dt, A, B, C)
    np.testing.assert_allclose(y[0, :, 0], [2, 3, 3.5, 3.75, 3.875, 3.9375], atol=1e-6)
    assert np.all(y[0, :, 1:] == 0)


# --------------------------------------------------------------------------
# Page "State Space Models (SSM)", section "Come funzionano gli SSM": for
# time-invariant parameters the recurrence equals a causal convolution of the
# input with the system's impulse response, from a zero initial state.  The
# page checks this on a 64-step, 16-state diagonal system with step 0.1 and
# the exact zero-order hold; only those sizes and its tolerance are taken
# from it (tests/golden/conv_demo.json).  The draws are this file's own.
# --------------------------------------------------------------------------
def _diag_system(seed, n):
    """Decay rates in [0.3, 2.0) (log-uniform), input and output gains
    N(0, 1): a stable diagonal system of n states."""
    r = _rng(seed)
    rate = np.exp(r.uniform(math.log(0.3), math.log(2.0), n))
    return (-rate).astype(np.float32), r.standard_normal(n), r.standard_normal(n), r


def _impulse_response(A, gain_in, gain_out, step, L):
    """h[k] = sum_n gain_out_n exp(k step A_n) gain_in_n, k = 0 .. L-1: the
    output k steps after a unit input, by the closed form of each state's
    geometric decay (no recurrence)."""
    k = np.arange(L, dtype=np.float64)[:, None]
    return (gain_out[None, :] * np.exp(k * step * A[None, :].astype(np.float64)) *
            gain_in[None, :]).sum(axis=1)


def _causal_convolution(h, x):
    """y = T x with T the lower-triangular Toeplitz matrix of h."""
    from scipy.linalg import toeplitz
    T = toeplitz(h, np.zeros_like(h))
    return T @ x


def test_recurrence_equals_convolution_diagonal(oracle_mod):
    """Each diagonal state becomes one head (P = N = 1, its own B/C group);
    the scan multiplies B by dt, so the exact zero-order-hold input gain
    (exp(step A) - 1) / A B is handed in divided by the step."""
    g = json.loads((GOLDEN / "conv_demo.json").read_text())
    L, Ns, step = g["seqlen"], g["state_size"], np.float32(g["delta"])
    A32, Bc, Cc, r = _diag_system(7, Ns)
    xs = r.standard_normal(L).astype(np.float32)
    s64, A64 = np.float64(step), A32.astype(np.float64)
    gain_in = np.expm1(s64 * A64) / A64 * Bc
    Bin = (gain_in / s64).astype(np.float32)
    x = np.repeat(xs[None, :, None, None], Ns, axis=2)                       # 1 L H 1
    dt = np.full((1, L, Ns), step, np.float32)
    Bm = np.broadcast_to(Bin[None, None, :, None], (1, L, Ns, 1)).copy()
    Cm = np.broadcast_to(Cc.astype(np.float32)[None, None, :, None], (1, L, Ns, 1)).copy()
    y_sel, _ = oracle_mod.forward(x, dt, A32, Bm, Cm)
    y_rec = y_sel[:, :, 0].sum(axis=0)
    # the convolution, from the gains the oracle actually consumed
    h = _impulse_response(A32, s64 * Bin.astype(np.float64),
                          Cc.astype(np.float32).astype(np.float64), s64, L)
    y_conv = _causal_convolution(h, xs.astype(np.float64))
    assert np.allclose(y_rec, y_conv, atol=g["compared_with_atol"])          # the page's check
    np.testing.assert_allclose(y_rec, y_conv, rtol=0, atol=1e-12 * np.abs(y_conv).max())


def test_recurrence_equals_convolution_scalar_decay(oracle_mod):
    """Scalar decay (one head, N = 16 entries fading together): the kernel is
    K_k = (C . B) dt a^k."""
    L, N = 64, 16
    r = _rng(8)
    a_cont = np.float32(-0.7)
    d = np.float32(0.1)
    Bv = r.standard_normal(N).astype(np.float32)
    Cv = r.standard_normal(N).astype(np.float32)
    xs = r.standard_normal(L).astype(np.float32)
    x = xs[None, :, None, None]
    dt = np.full((1, L, 1), d, np.float32)
    Bm = np.broadcast_to(Bv[None, None, None, :], (1, L, 1, N)).copy()
    Cm = np.broadcast_to(Cv[None, None, None, :], (1, L, 1, N)).copy()
    y, _ = oracle_mod.forward(x, dt, np.array([a_cont]), Bm, Cm)
    a = math.exp(float(d) * float(a_cont))
    cb = float(np.dot(Cv.astype(np.float64), Bv.astype(np.float64)))
    K = cb * float(d) * a ** np.arange(L)
    y_conv = np.array([np.dot(K[: t + 1][::-1], xs[: t + 1].astype(np.float64)) for t in range(L)])
    np.testing.assert_allclose(y[0, :, 0], y_conv, rtol=0, atol=1e-12 * np.abs(y_conv).max())


# --------------------------------------------------------------------------
# Page "Mamba-2 (2024): SSM e attention sono la stessa cosa", section "Due modi
# di guardare la stessa matrice": the whole layer is multiplication by one
# lower-triangular semiseparable matrix M (a low-rank description).
# --------------------------------------------------------------------------
def _brute_force_M(dt, A, B, C):
    """M[i, j] = (C_i . B_j) dt_j exp(sum_{k=j+1..i} dt_k A) for j <= i."""
    L = dt.shape[0]
    M = np.zeros((L, L))
    for i in range(L):
        for j in range(i + 1):
            decay = math.exp(sum(float(dt[k]) * float(A) for k in range(j + 1, i + 1)))
            M[i, j] = float(np.dot(C[i].astype(np.float64), B[j].astype(np.float64))) * float(dt[j]) * decay
    return M


def test_materialised_semiseparable_matrix(oracle_mod):
    c = _rand_case(11, batch=2, L=36, H=4, P=3, N=4, G=2)
    y, fin = oracle_mod.forward(**c)
    H, G = 4, 2
    for b in range(2):
        for h in range(H):
            g = h // (H // G)
            M = _brute_force_M(c["dt"][b, :, h], c["A"][h], c["B"][b, :, g], c["C"][b, :, g])
            xh = c["x"][b, :, h].astype(np.float64)                     # L x P
            carried = np.array([math.exp(sum(float(c["dt"][b, k, h]) * float(c["A"][h]) for k in range(i + 1)))
                                for i in range(36)])
            h0 = c["init"][b, h].astype(np.float64)                     # P x N
            ref = M @ xh + float(c["D"][h]) * xh + carried[:, None] * (c["C"][b, :, g].astype(np.float64) @ h0.T)
            k = b * H + h
            np.testing.assert_allclose(y[k], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_operator_matrix_is_lower_triangular_low_rank(oracle_mod):
    """Probe the oracle with unit impulses to read out its operator matrix;
    it must equal the brute-force M, be zero above the diagonal, and every
    off-diagonal block M[r:, :r] must have rank <= N."""
    L, N = 40, 3
    c = _rand_case(12, batch=1, L=L, H=1, P=1, N=N, G=1, with_init=False, with_D=False)
    cols = []
    for j in range(L):
        x = np.zeros((1, L, 1, 1), np.float32)
        x[0, j, 0, 0] = 1.0
        y, _ = oracle_mod.forward(x, c["dt"], c["A"], c["B"], c["C"])
        cols.append(y[0, :, 0])
    Mo = np.stack(cols, axis=1)
    Mb = _brute_force_M(c["dt"][0, :, 0], c["A"][0], c["B"][0, :, 0], c["C"][0, :, 0])
    np.testing.assert_allclose(Mo, Mb, rtol=0, atol=1e-13 * np.abs(Mb).max())
    assert np.all(np.triu(Mo, 1) == 0)
    for rr in range(1, L):
        s = np.linalg.svd(Mo[rr:, :rr], compute_uv=False)
        if s.size > N:
            assert np.all(s[N:] <= 1e-10 * s[0])


# --------------------------------------------------------------------------
# Page "State Space Model", section "Due strade, una meta": with a scalar
# transition the SSM is masked linear attention without softmax; with A = 0
# nothing fades and the weights are plain C_i . B_j dt_j.
# --------------------------------------------------------------------------
def test_zero_decay_is_causal_linear_attention(oracle_mod):
    c = _rand_case(13, batch=1, L=50, H=2, P=4, N=6, G=1, with_init=False)
    c["A"] = np.zeros_like(c["A"])
    y, _ = oracle_mod.forward(**c)
    Bm, Cm = c["B"][0, :, 0].astype(np.float64), c["C"][0, :, 0].astype(np.float64)
    scores = np.tril(Cm @ Bm.T)                                  # causal mask, no softmax
    for h in range(2):
        v = c["dt"][0, :, h].astype(np.float64)[:, None] * c["x"][0, :, h].astype(np.float64)
        ref = scores @ v + float(c["D"][h]) * c["x"][0, :, h].astype(np.float64)
        np.testing.assert_allclose(y[h], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


# --------------------------------------------------------------------------
# Page "State Space Model", section "Un sistema che riassume il passato":
# Delta -> 0 keeps the state and ignores the input; a large Delta forgets the
# past and the current input dominates.
# --------------------------------------------------------------------------
def test_zero_step_keeps_state(oracle_mod):
    c = _rand_case(14, batch=2, L=20, H=2, P=3, N=4, G=1)
    c["dt"] = np.zeros_like(c["dt"])
    y, fin = oracle_mod.forward(**c)
    for b in range(2):
        for h in range(2):
            k = b * 2 + h
            h0 = c["init"][b, h].astype(np.float64)
            assert np.array_equal(fin[k], h0)
            ref = c["C"][b, :, 0].astype(np.float64) @ h0.T + float(c["D"][h]) * c["x"][b, :, h].astype(np.float64)
            np.testing.assert_allclose(y[k], ref, rtol=0, atol=1e-13 * np.abs(ref).max())


def test_huge_step_is_memoryless(oracle_mod):
    c = _rand_case(15, batch=1, L=20, H=2, P=3, N=4, G=1)
    c["dt"] = np.full_like(c["dt"], 1e4)
    y, fin = oracle_mod.forward(**c)
    for h in range(2):
        Bm, Cm = c["B"][0, :, 0].astype(np.float64), c["C"][0, :, 0].astype(np.float64)
        x = c["x"][0, :, h].astype(np.float64)
        cb = np.sum(Cm * Bm, axis=1)
        ref = 1e4 * x * cb[:, None] + float(c["D"][h]) * x
        np.testing.assert_allclose(y[h], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_skip_term_alone_when_B_is_zero(oracle_mod):
    c = _rand_case(16, batch=1, L=10, H=3, P=2, N=3, G=1, with_init=False)
    c["B"] = np.zeros_like(c["B"])
    y, fin = oracle_mod.forward(**c)
    for h in range(3):
        assert np.array_equal(y[h], float(c["D"][h]) * c["x"][0, :, h].astype(np.float64))
    assert np.all(fin == 0)


# --------------------------------------------------------------------------
# Page "State Space Model", section "Un sistema che riassume il passato": steps
# compose associatively (so a sequence may be cut anywhere and resumed from the
# state), and the model is run step by step to generate.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("m", [1, 17, 39])
def test_split_sequence_resume(oracle_mod, m):
    c = _rand_case(17, batch=2, L=40, H=4, P=3, N=5, G=2)
    y_full, fin_full = oracle_mod.forward(**c)
    first = {k: (v[:, :m] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
    y1, f1 = oracle_mod.forward(**first)
    second = {k: (v[:, m:] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
    second["init"] = f1.reshape(2, 4, 3, 5).astype(np.float32)
    y2, f2 = oracle_mod.forward(**second)
    # the hand-over rounds the fp64 state to fp32; compare at that precision
    np.testing.assert_allclose(y1, y_full[:, :m], rtol=0, atol=0)
    np.testing.assert_allclose(y2, y_full[:, m:], rtol=0, atol=1e-6 * np.abs(y_full).max())
    np.testing.assert_allclose(f2, fin_full, rtol=0, atol=1e-6 * np.abs(fin_full).max())


def test_step_by_step_equals_forward(oracle_mod):
    c = _rand_case(18, batch=2, L=12, H=4, P=3, N=5, G=2)
    y, fin = oracle_mod.forward(**c)
    st = c["init"].astype(np.float64).copy()
    for t in range(12):
        yt = oracle_mod.step(st, c["x"][:, t], c["dt"][:, t], c["A"], c["B"][:, t], c["C"][:, t], c["D"])
        np.testing.assert_allclose(yt.reshape(8, 3), y[:, t], rtol=0, atol=1e-13 * np.abs(y).max())
    np.testing.assert_allclose(st.reshape(8, 3, 5), fin, rtol=0, atol=1e-13 * np.abs(fin).max())


# --------------------------------------------------------------------------
# Head -> group map and layouts: the pages are silent (our convention).  These
# keep the oracle internally consistent; parity of the convention itself is
# unpinned by the pages.
# --------------------------------------------------------------------------
def test_group_permutation_equivariance(oracle_mod):
    H, G = 6, 3
    c = _rand_case(19, batch=1, L=15, H=H, P=2, N=3, G=G)
    y, fin = oracle_mod.forward(**c)
    gperm = np.array([2, 0, 1])
    hperm = np.concatenate([np.arange(2 * g, 2 * g + 2) for g in gperm])
    c2 = dict(c)
    c2["B"], c2["C"] = c["B"][:, :, gperm], c["C"][:, :, gperm]
    for k in ("x", "dt"):
        c2[k] = c[k][:, :, hperm]
    c2["A"], c2["D"] = c["A"][hperm], c["D"][hperm]
    c2["init"] = c["init"][:, hperm]
    y2, fin2 = oracle_mod.forward(**c2)
    assert np.array_equal(y2, y[hperm])
    assert np.array_equal(fin2, fin[hperm])


def test_groups_matter(oracle_mod):
    """Heads of different groups must see different B/C: swapping the two
    groups' B changes the output of every head."""
    c = _rand_case(20, batch=1, L=10, H=4, P=2, N=3, G=2, with_init=False)
    y, _ = oracle_mod.forward(**c)
    c2 = dict(c)
    c2["B"] = c["B"][:, :, ::-1].copy()
    y2, _ = oracle_mod.forward(**c2)
    for h in range(4):
        assert not np.allclose(y[h], y2[h])


def test_bf16_storage_is_widened_exactly(oracle_mod):
    import torch
    c = _rand_case(21, batch=1, L=9, H=2, P=3, N=4, G=1)
    xb = torch.from_numpy(c["x"]).to(torch.bfloat16)
    Bb = torch.from_numpy(c["B"]).to(torch.bfloat16)
    Cb = torch.from_numpy(c["C"]).to(torch.bfloat16)
    c_bf = dict(c, x=xb, B=Bb, C=Cb)
    c_up = dict(c, x=xb.float().numpy(), B=Bb.float().numpy(), C=Cb.float().numpy())
    y1, f1 = oracle_mod.forward(**c_bf)
    y2, f2 = oracle_mod.forward(**c_up)
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)


def test_selected_heads_and_token_window(oracle_mod):
    c = _rand_case(22, batch=2, L=30, H=4, P=3, N=5, G=2)
    y, fin = oracle_mod.forward(**c)
    ys, fs = oracle_mod.forward(**c, bh=[(1, 3), (0, 2)], t_range=(7, 19))
    assert np.array_equal(ys[0], y[1 * 4 + 3, 7:19]) and np.array_equal(ys[1], y[2, 7:19])
    assert np.array_equal(fs[0], fin[7]) and np.array_equal(fs[1], fin[2])


# --------------------------------------------------------------------------
# Page "Mamba-2 (2024): SSM e attention sono la stessa cosa", section "Il
# trucco a blocchi": cutting the sequence into blocks, quadratic inside and a
# carried state between, computes the same result for any block size.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Q", [1, 7, 16, 64, 100])
def test_chunk_stages_match_recurrence(oracle_mod, Q):
    from oracle import stages
    c = _rand_case(23, batch=2, L=100, H=4, P=3, N=5, G=2)
    y_ref, fin_ref = oracle_mod.forward_full(**c)
    y, fin, Acs, S, Hin = stages.forward(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["init"], Q)
    np.testing.assert_allclose(y, y_ref, rtol=0, atol=1e-12 * np.abs(y_ref).max())
    np.testing.assert_allclose(fin, fin_ref, rtol=0, atol=1e-12 * np.abs(fin_ref).max())
    # block-end states from zero, chained, reproduce the recurrence's state at
    # every block boundary
    for cidx in range(1, Hin.shape[2]):
        t_end = cidx * Q
        _, f_pref = oracle_mod.forward(**{k: (v[:, :t_end] if k in ("x", "dt", "B", "C") else v)
                                         for k, v in c.items()})
        np.testing.assert_allclose(Hin[:, :, cidx].reshape(-1, 3, 5), f_pref, rtol=0,
                                   atol=1e-12 * np.abs(f_pref).max())
        if cidx > 3:
            break


def test_chunk_cumsum_definition():
    from oracle import stages
    dt = np.arange(1, 11, dtype=np.float32).reshape(1, 10, 1) / 10
    A = np.array([-2.0], np.float32)
    Acs = stages.chunk_cumsum(dt, A, 4)
    assert Acs.shape == (1, 1, 3, 4)
    np.testing.assert_allclose(Acs[0, 0, 0], -2 * np.cumsum(dt[0, :4, 0]), rtol=1e-6)
    np.testing.assert_allclose(Acs[0, 0, 2], [-1.8, -3.8, -3.8, -3.8], rtol=1e-6)


# --------------------------------------------------------------------------
# Page "State Space Models (SSM)" (ultralytics.com glossary), section "Come
# funzionano gli SSM": the exact zero-order hold Bbar = (Abar - 1) / A B used
# by its recurrent-versus-convolutional demonstration.
# --------------------------------------------------------------------------
def test_zoh_convolution_demo(oracle_mod):
    """The same check with the oracle's own zero-order hold: B is handed in
    as drawn, and the recurrence must equal the causal convolution with the
    impulse response built from the exact hold's input gain (fp64)."""
    g = json.loads((GOLDEN / "conv_demo.json").read_text())
    L, Ns, step = g["seqlen"], g["state_size"], np.float32(g["delta"])
    A32, B64, C64, r = _diag_system(17, Ns)
    B32, C32 = B64.astype(np.float32), C64.astype(np.float32)
    xs = r.standard_normal(L).astype(np.float32)
    x = np.repeat(xs[None, :, None, None], Ns, axis=2)
    dt = np.full((1, L, Ns), step, np.float32)
    Bm = np.broadcast_to(B32[None, None, :, None], (1, L, Ns, 1)).copy()
    Cm = np.broadcast_to(C32[None, None, :, None], (1, L, Ns, 1)).copy()
    y_sel, _ = oracle_mod.forward(x, dt, A32, Bm, Cm, zoh=True)
    y_rec = y_sel[:, :, 0].sum(axis=0)
    A64, s64 = A32.astype(np.float64), np.float64(step)
    gain_in = np.expm1(s64 * A64) / A64 * B32.astype(np.float64)
    h = _impulse_response(A32, gain_in, C32.astype(np.float64), s64, L)
    y_conv = _causal_convolution(h, xs.astype(np.float64))
    assert np.allclose(y_rec, y_conv, atol=g["compared_with_atol"])          # the page's check
    np.testing.assert_allclose(y_rec, y_conv, rtol=0, atol=1e-12 * np.abs(y_conv).max())


@pytest.mark.parametrize("d", [0.05, 0.7, 3.0])
def test_zoh_step_response_closed_form(oracle_mod, d):
    """Constant input x = 1 from an empty state, one scalar decay: with the
    zero-order hold each state entry is -B/A (1 - exp(A d (t + 1))) after
    token t, so the level it settles at, -B/A, does not depend on the step
    size (the hold keeps the continuous system's steady state); the plain
    dt B form settles at d B / (1 - exp(A d)) instead."""
    L, N = 40, 6
    r = _rng(18)
    A = np.array([-0.9], np.float32)
    Bv = r.standard_normal(N).astype(np.float32)
    Cv = r.standard_normal(N).astype(np.float32)
    x = np.ones((1, L, 1, 1), np.float32)
    dt = np.full((1, L, 1), np.float32(d), np.float32)
    Bm = np.broadcast_to(Bv[None, None, None, :], (1, L, 1, N)).copy()
    Cm = np.broadcast_to(Cv[None, None, None, :], (1, L, 1, N)).copy()
    y, fin = oracle_mod.forward(x, dt, A, Bm, Cm, zoh=True)
    a64, d64 = float(A[0]), float(np.float32(d))
    B64, C64 = Bv.astype(np.float64), Cv.astype(np.float64)
    t = np.arange(L)
    expect = float(np.dot(C64, -B64 / a64)) * (1.0 - np.exp(a64 * d64 * (t + 1)))
    np.testing.assert_allclose(y[0, :, 0], expect, rtol=0, atol=1e-13)
    np.testing.assert_allclose(fin[0, 0], -B64 / a64 * (1.0 - math.exp(a64 * d64 * L)), rtol=1e-13, atol=0)
    y_e, _ = oracle_mod.forward(x, dt, A, Bm, Cm)
    steady_e = float(np.dot(C64, B64)) * d64 / (1.0 - math.exp(a64 * d64))
    assert abs(y_e[0, -1, 0] - steady_e * (1.0 - math.exp(a64 * d64 * L))) < 1e-12


def test_zoh_small_step_limit_and_zero_decay(oracle_mod):
    """expm1(dt A) / A -> dt as dt A -> 0: with A = 0 the two forms are the
    same computation, and for tiny dt A they agree to about |dt A| / 2."""
    c = _rand_case(19, L=30, H=3, G=1)
    c0 = dict(c, A=np.zeros(3, np.float32))
    y_z, f_z = oracle_mod.forward(**c0, zoh=True)
    y_e, f_e = oracle_mod.forward(**c0)
    assert np.array_equal(y_z, y_e) and np.array_equal(f_z, f_e)
    cs = dict(c, dt=(c["dt"] * 1e-4).astype(np.float32))
    y_z, _ = oracle_mod.forward(**cs, zoh=True)
    y_e, _ = oracle_mod.forward(**cs)
    bound = float(np.max(np.abs(cs["dt"]))) * float(np.max(np.abs(c["A"]))) * np.abs(y_e).max()
    assert np.max(np.abs(y_z - y_e)) <= bound
    assert np.max(np.abs(y_z - y_e)) > 0


def test_zoh_step_equals_forward(oracle_mod):
    """The decode step with the zero-order hold, token by token, reproduces the
    whole-sequence recurrence with it."""
    c = _rand_case(20, batch=2, L=12, H=4, P=3, N=5, G=2)
    y_full, fin_full = oracle_mod.forward(**c, zoh=True)
    state = np.ascontiguousarray(c["init"].astype(np.float64))
    ys = []
    for t in range(12):
        ys.append(oracle_mod.step(state, c["x"][:, t], c["dt"][:, t], c["A"], c["B"][:, t],
                                  c["C"][:, t], c["D"], zoh=True))
    y_steps = np.stack(ys, axis=1)                              # b t h p
    y_ref = y_full.reshape(2, 4, 12, 3).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(y_steps, y_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(state, fin_full.reshape(2, 4, 3, 5), rtol=0, atol=1e-12)


@pytest.mark.parametrize("K", [1, 2, 3, 5, 8, 40])
def test_two_level_recurrence_equals_the_chain(K):
    """The two-level form (runs of K blocks scanned from zero, a chain over
    the runs, entering states recombined) gives the same entering states and
    final state as the plain chain between blocks, for run lengths that
    divide the block count, leave a short last run, and exceed it."""
    from oracle import stages
    rng = np.random.default_rng(7)
    batch, H, nc, P, N = 2, 3, 11, 4, 5
    S = rng.standard_normal((batch, H, nc, P, N))
    Acs = -np.abs(rng.standard_normal((batch, H, nc, 6))).cumsum(axis=3) * 0.3
    init = rng.standard_normal((batch, H, P, N))
    Hin, fin = stages.state_passing(S, Acs, init)
    T, lam, rdec = stages.run_states(S, Acs, K)
    Hr, fin2 = stages.run_passing(T, rdec, K, init)
    Hin2 = stages.runs_entering_states(T, Hr, lam, K)
    assert np.allclose(Hin2, Hin, rtol=1e-12, atol=1e-12)
    assert np.allclose(fin2, fin, rtol=1e-12, atol=1e-12)
    # a run of one block is the plain chain: T is S and Hr is Hin
    if K == 1:
        assert np.allclose(T, S) and np.allclose(Hr, Hin)
    # the run decays sum the blocks' decays
    assert np.allclose(rdec.sum(axis=2), Acs[:, :, :, -1].sum(axis=2))
