"""Pins of oracle/layer.py (the steps around the scan) to facts that do not
come from the oracle's own formulas: identities of silu and softplus, special
values, unit-tap filters, causality and numpy's own convolution."""
import math

import numpy as np

from oracle import layer


def test_silu_and_softplus_odd_parts():
    """silu(v) - silu(-v) = v and softplus(v) - softplus(-v) = v for every v
    (both are v times / plus a function whose odd part is v / 2)."""
    v = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(layer.silu(v) - layer.silu(-v), v, rtol=0, atol=1e-13)
    np.testing.assert_allclose(layer.softplus(v) - layer.softplus(-v), v, rtol=0, atol=1e-12)


def test_special_values_and_limits():
    assert layer.silu(0.0) == 0.0
    assert layer.softplus(0.0) == math.log(2.0)
    assert abs(layer.silu(40.0) - 40.0) < 1e-12 and abs(layer.silu(-40.0)) < 1e-15
    assert abs(layer.softplus(40.0) - 40.0) < 1e-12 and 0.0 < layer.softplus(-40.0) < 1e-17
    # silu(1) = 1 / (1 + 1/e) = e / (e + 1)
    assert abs(layer.silu(1.0) - math.e / (math.e + 1.0)) < 1e-15


def test_unit_tap_filters():
    """The tap on the current token alone is the identity; the oldest tap alone
    shifts the sequence by K - 1 tokens (zeros enter at the start); a bias
    adds itself."""
    r = np.random.default_rng(1)
    u = r.standard_normal((2, 9, 5))
    K = 4
    w = np.zeros((5, K)); w[:, K - 1] = 1.0
    np.testing.assert_array_equal(layer.causal_conv(u, w), u)
    w = np.zeros((5, K)); w[:, 0] = 1.0
    shifted = np.zeros_like(u); shifted[:, K - 1:] = u[:, : 9 - (K - 1)]
    np.testing.assert_array_equal(layer.causal_conv(u, w), shifted)
    b = r.standard_normal(5)
    np.testing.assert_allclose(layer.causal_conv(u, w, b), shifted + b, rtol=0, atol=1e-15)


def test_causality_and_numpy_convolve():
    """Changing token t changes no output before t; each channel equals
    numpy.convolve of the input with its filter (taps reversed), cut to the
    sequence length."""
    r = np.random.default_rng(2)
    u = r.standard_normal((1, 30, 3))
    w = r.standard_normal((3, 4))
    out = layer.causal_conv(u, w)
    u2 = u.copy(); u2[0, 17] += 5.0
    out2 = layer.causal_conv(u2, w)
    assert np.array_equal(out[0, :17], out2[0, :17]) and not np.array_equal(out[0, 17], out2[0, 17])
    for c in range(3):
        ref = np.convolve(u[0, :, c], w[c, ::-1])[:30]
        np.testing.assert_allclose(out[0, :, c], ref, rtol=0, atol=1e-13)


def test_layer_in_split_and_layer_out():
    """layer_in splits the convolved channels in the order x (head-major),
    B, C, and adds the step bias before softplus; layer_out gates by silu."""
    r = np.random.default_rng(3)
    H, P, G, N, K = 2, 3, 1, 4, 2
    Cd = H * P + 2 * G * N
    xbc = r.standard_normal((1, 5, Cd))
    w = np.zeros((Cd, K)); w[:, K - 1] = 1.0      # identity filter
    dt_raw = r.standard_normal((1, 5, H)); dt_bias = np.array([0.5, -1.0])
    x, Bm, Cm, dt = layer.layer_in(xbc, w, None, dt_raw, dt_bias, H, P, G, N)
    s = layer.silu(xbc)
    np.testing.assert_array_equal(x[0, :, 1, 2], s[0, :, 1 * P + 2])
    np.testing.assert_array_equal(Bm[0, :, 0, 3], s[0, :, H * P + 3])
    np.testing.assert_array_equal(Cm[0, :, 0, 1], s[0, :, H * P + N + 1])
    np.testing.assert_array_equal(dt, layer.softplus(dt_raw + dt_bias))
    y = r.standard_normal((1, 5, H * P))
    np.testing.assert_array_equal(layer.layer_out(y, np.zeros_like(y)), np.zeros_like(y))
    # silu(60) = 60 (1 - 1e-26 or so); silu(1) = e / (e + 1)
    np.testing.assert_allclose(layer.layer_out(y, np.full_like(y, 60.0)), 60.0 * y, rtol=1e-15, atol=0)
    np.testing.assert_allclose(layer.layer_out(y, np.ones_like(y)), y * math.e / (math.e + 1.0),
                               rtol=1e-15, atol=0)
