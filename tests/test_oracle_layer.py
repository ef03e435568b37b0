"""Pins for the layer oracle (oracle/layer.py), CPU only: the short
convolution against numpy's convolution, closed forms of Swish and the L2 and
RMS normalisations, continuation through the carried state, and a planted
mistake (reversed taps) that the convolution pin catches."""
import numpy as np
import pytest

from oracle import layer


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def test_conv_matches_numpy_convolve():
    """Per channel, before Swish and L2: c_t = sum_i w[W-1-i] x_{t-i}, which is
    numpy's full convolution of x with the reversed taps, truncated."""
    rng = np.random.default_rng(0)
    T, H, d, W = 23, 2, 5, 4
    x = rng.standard_normal((T, H, d))
    w = rng.standard_normal((H, d, W))
    y, _ = layer.shortconv_swish_l2(x, w, [0, T])
    c = np.zeros((T, H, d))
    for h in range(H):
        for ch in range(d):
            c[:, h, ch] = np.convolve(x[:, h, ch], w[h, ch, ::-1])[:T]
    s = c * sig(c)
    exp = s / np.sqrt((s * s).sum(-1, keepdims=True) + layer.EPS_L2)
    np.testing.assert_allclose(y, exp, rtol=1e-12, atol=1e-14)


def test_width_one_unit_weight_is_swish_then_l2():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 3, 8))
    y, st = layer.shortconv_swish_l2(x, np.ones((3, 8, 1)), [0, 4, 9])
    s = x * sig(x)
    np.testing.assert_allclose(y, s / np.sqrt((s * s).sum(-1, keepdims=True) + 1e-6),
                               rtol=1e-13)
    assert st.shape == (2, 3, 8, 0)


def test_norm_closed_form():
    """|y_t| = sqrt(S / (S + eps)), S = |Swish(c)|^2: at most 1."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((30, 1, 16)) * 3
    w = rng.standard_normal((1, 16, 3))
    y, _ = layer.shortconv_swish_l2(x, w, [0, 30])
    nrm = np.linalg.norm(y, axis=-1)
    assert np.all(nrm <= 1.0) and np.all(nrm > 0.99)


@pytest.mark.parametrize("cut", [1, 2, 3, 17])
def test_state_continuation(cut):
    """Running a sequence in two calls with the state carried equals one call,
    outputs and final state (includes pieces shorter than W - 1)."""
    rng = np.random.default_rng(3)
    T, H, d, W = 20, 2, 6, 4
    x = rng.standard_normal((T, H, d))
    w = rng.standard_normal((H, d, W))
    s0 = rng.standard_normal((1, H, d, W - 1))
    y, s_end = layer.shortconv_swish_l2(x, w, [0, T], s0)
    y1, s1 = layer.shortconv_swish_l2(x[:cut], w, [0, cut], s0)
    y2, s2 = layer.shortconv_swish_l2(x[cut:], w, [0, T - cut], s1)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(s2, s_end)


def test_state_out_short_sequence_and_empty():
    """The carried state is the last W - 1 inputs of [state_in, sequence]."""
    d, W = 2, 4
    s0 = np.arange(1 * 1 * d * (W - 1), dtype=float).reshape(1, 1, d, W - 1) + 100
    x = np.array([[[1.0, 2.0]]])          # one token
    _, st = layer.shortconv_swish_l2(x, np.ones((1, d, W)), [0, 1], s0)
    np.testing.assert_array_equal(st[0, 0], np.stack([s0[0, 0, :, 1], s0[0, 0, :, 2],
                                                      x[0, 0]], axis=-1))
    _, st_e = layer.shortconv_swish_l2(np.zeros((0, 1, d)), np.ones((1, d, W)), [0, 0], s0)
    np.testing.assert_array_equal(st_e, s0)


def test_rmsnorm_gate_hand_example():
    o = np.array([[[3.0, 4.0]]])
    eps = 1e-6
    y = layer.rmsnorm_gate(o, np.array([[[0.0, np.inf]]]), np.array([1.0, 2.0]), eps)
    r = np.sqrt(12.5 + eps)
    np.testing.assert_allclose(y[0, 0], [3.0 / r * 0.5, 4.0 / r * 2.0], rtol=1e-15)


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((7, 3, 16))
    y1 = layer.rmsnorm_gate(o, None, None, 0.0)
    y2 = layer.rmsnorm_gate(37.5 * o, None, None, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    np.testing.assert_allclose(np.sqrt((y1 * y1).mean(-1)), 1.0, rtol=1e-13)


def _mutant_reversed_taps(x, w, cu):
    return layer.shortconv_swish_l2(x, w[:, :, ::-1], cu)


def test_planted_reversed_taps_is_caught():
    rng = np.random.default_rng(5)
    T, H, d, W = 12, 1, 4, 3
    x = rng.standard_normal((T, H, d))
    w = rng.standard_normal((H, d, W))
    y_m, _ = _mutant_reversed_taps(x, w, [0, T])
    c = np.stack([np.convolve(x[:, 0, ch], w[0, ch, ::-1])[:T] for ch in range(d)], -1)
    s = c * sig(c)
    exp = s / np.sqrt((s * s).sum(-1, keepdims=True) + 1e-6)
    assert np.abs(y_m[:, 0] - exp).max() > 1e-2
