"""Pins for the prologue / epilogue oracle (oracle/layer.py), CPU only.

Each pin checks the oracle against something other than itself: a library
routine it does not call (numpy.convolve for the causal convolution,
scipy.special.expit for the sigmoid), closed forms (the norm of an
L2-normalised vector, RMSNorm of a constant vector, sigmoid(0) = 1/2, the
decay bound), and invariants (splitting a sequence with the cached
convolution history, resets at packed-sequence boundaries, scale invariance
of the norms).  test_oracle_layer_mutants.py plants mistakes in copies of the
oracle and checks that these pins catch each one.

Every pin takes the oracle module as `L`, so the mutant test can run the same
pins against a broken copy.
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import layer as ORACLE


def _rng(seed):
    return np.random.default_rng(seed)


def pin_sigmoid_and_swish_against_expit(L):
    z = np.linspace(-30.0, 30.0, 241)
    assert np.allclose(L.sigmoid(z), expit(z), rtol=1e-14, atol=1e-300)
    assert np.allclose(L.swish(z), z * expit(z), rtol=1e-13, atol=1e-300)
    assert L.sigmoid(0.0) == 0.5 and L.swish(0.0) == 0.0


def pin_conv_against_numpy_convolve(L):
    g = _rng(1)
    T, C = 37, 5
    x = g.standard_normal((T, C))
    w = g.standard_normal((C, 4))           # asymmetric taps
    y, hist = L.short_conv(x, w)
    for c in range(C):
        # y[t] = sum_j w[c, 3 - j] x[t - j]: a full convolution with the taps reversed
        ref = np.convolve(x[:, c], w[c, ::-1])[:T]
        assert np.allclose(y[:, c], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(hist[0], x[-3:])


def pin_conv_special_weights(L):
    g = _rng(2)
    x = g.standard_normal((20, 3))
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (3, 1))
    y, _ = L.short_conv(x, ident)
    assert np.array_equal(y, x)
    lag3 = np.tile([1.0, 0.0, 0.0, 0.0], (3, 1))
    y, _ = L.short_conv(x, lag3)
    assert np.array_equal(y[3:], x[:-3]) and not y[:3].any()


def pin_conv_split_with_history_equals_whole(L):
    g = _rng(3)
    T, C = 50, 4
    x = g.standard_normal((T, C))
    w = g.standard_normal((C, 4))
    h0 = g.standard_normal((1, 3, C))
    y, h = L.short_conv(x, w, history=h0)
    for cut in (1, 2, 3, 17):
        y1, h1 = L.short_conv(x[:cut], w, history=h0)
        y2, h2 = L.short_conv(x[cut:], w, history=h1)
        assert np.allclose(np.concatenate([y1, y2]), y, rtol=1e-12, atol=1e-12)
        assert np.array_equal(h2, h)
    # a one-token sequence shifts the history by one
    _, h1 = L.short_conv(x[:1], w, history=h0)
    assert np.array_equal(h1[0], np.concatenate([h0[0, 1:], x[:1]]))


def pin_conv_resets_at_sequence_boundaries(L):
    g = _rng(4)
    lengths = [5, 1, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    C = 3
    x = g.standard_normal((cu[-1], C))
    w = g.standard_normal((C, 4))
    hist = g.standard_normal((len(lengths), 3, C))
    y, h = L.short_conv(x, w, cu_seqlens=cu, history=hist)
    for n in range(len(lengths)):
        yn, hn = L.short_conv(x[cu[n]:cu[n + 1]], w, history=hist[n:n + 1])
        assert np.allclose(y[cu[n]:cu[n + 1]], yn, rtol=1e-12, atol=1e-12)
        assert np.array_equal(h[n], hn[0])
    assert np.array_equal(h[2], hist[2])      # an empty sequence keeps its history


def pin_l2_normalize(L):
    g = _rng(5)
    x = g.standard_normal((6, 4, 16)) * np.array([1e-1, 1.0, 10.0, 1e3])[None, :, None]
    eps = 1e-6
    y = L.l2_normalize(x, eps)
    n2 = np.sum(x * x, axis=-1)
    # |y| = |x| / sqrt(|x|^2 + eps), per (token, head)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.sqrt(n2 / (n2 + eps)), rtol=1e-12)
    # direction kept
    assert np.allclose(y * np.linalg.norm(x, axis=-1, keepdims=True) /
                       np.linalg.norm(y, axis=-1, keepdims=True), x, rtol=1e-12)


def pin_log_decay_bound_and_bias(L):
    g = _rng(6)
    a = g.standard_normal((7, 3, 8)) * 4
    bias = g.standard_normal((3, 8))
    d = L.log_decay(a, bias)
    assert d.shape == a.shape
    assert (d < 0).all() and (d > -5).all()
    assert np.allclose(d, -5.0 * expit(a + bias[None]), rtol=1e-14)
    assert L.log_decay(np.zeros((1, 1, 1)), np.zeros((1, 1)))[0, 0, 0] == -2.5
    # a larger logit decays more (log alpha decreasing in a + bias)
    assert L.log_decay(np.array([[[1.0]]]), np.zeros((1, 1))) < \
        L.log_decay(np.array([[[0.0]]]), np.zeros((1, 1)))


def pin_write_strength(L):
    b = np.linspace(-20, 20, 81).reshape(9, 9)
    assert np.allclose(L.write_strength(b), expit(b), rtol=1e-14)
    assert L.write_strength(np.zeros(1))[0] == 0.5


def pin_head_rmsnorm(L):
    g = _rng(7)
    eps = 1e-5
    # a constant vector c over D channels: c / sqrt(c^2 + eps) * w
    D = 16
    c = np.array([0.5, -2.0, 3.0])
    o = np.repeat(c[None, :, None], D, axis=2)            # [1, 3, D]
    w = g.standard_normal((3, D))
    y = L.head_rmsnorm(o, w, eps)
    assert np.allclose(y, (c / np.sqrt(c * c + eps))[None, :, None] * w[None], rtol=1e-12)
    # per-head statistics: heads at very different scales come out at unit RMS
    o = g.standard_normal((5, 3, D)) * np.array([1e-1, 1.0, 1e2])[None, :, None]
    y = L.head_rmsnorm(o, np.ones((3, D)), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)


def pin_epilogue_gate(L):
    g = _rng(8)
    o = g.standard_normal((4, 2, 8))
    w = g.standard_normal((2, 8))
    base = L.head_rmsnorm(o, w, 1e-5)
    assert np.allclose(L.epilogue(o, np.full_like(o, 50.0), w), base, rtol=1e-12)
    assert np.allclose(L.epilogue(o, np.zeros_like(o), w), 0.5 * base, rtol=1e-14)
    gg = g.standard_normal(o.shape)
    assert np.allclose(L.epilogue(o, gg, w), base * expit(gg), rtol=1e-12)


def pin_prologue_composition(L):
    """With identity taps the prologue is plain elementwise work; the
    convolution history lands in [N, tensor, token, H, D]."""
    g = _rng(9)
    T, H, D = 11, 2, 8
    lengths = [4, 7]
    cu = np.array([0, 4, 11])
    xq, xk, xv, a = (g.standard_normal((T, H, D)) for _ in range(4))
    b = g.standard_normal((T, H))
    ident = np.zeros((3, H, D, 4))
    ident[..., 3] = 1.0
    bias = g.standard_normal((H, D))
    q, k, v, la, beta, st = L.prologue(xq, xk, xv, a, b, ident, bias, cu_seqlens=cu)

    def sw(x):
        return x * expit(x)

    def nrm(x):
        return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)

    assert np.allclose(q, nrm(sw(xq)), rtol=1e-12)
    assert np.allclose(k, nrm(sw(xk)), rtol=1e-12)
    assert np.allclose(v, sw(xv), rtol=1e-12)
    assert np.allclose(la, -5 * expit(a + bias[None]), rtol=1e-12)
    assert np.allclose(beta, expit(b), rtol=1e-12)
    assert st.shape == (2, 3, 3, H, D)
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        for i, x in enumerate((xq, xk, xv)):
            assert np.array_equal(st[n, i], x[e - 3:e])
    del lengths


PINS = [pin_sigmoid_and_swish_against_expit, pin_conv_against_numpy_convolve,
        pin_conv_special_weights, pin_conv_split_with_history_equals_whole,
        pin_conv_resets_at_sequence_boundaries, pin_l2_normalize, pin_log_decay_bound_and_bias,
        pin_write_strength, pin_head_rmsnorm, pin_epilogue_gate, pin_prologue_composition]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_layer_oracle_pin(pin):
    pin(ORACLE)
