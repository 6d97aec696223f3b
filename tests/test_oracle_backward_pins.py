"""Pins for the backward oracle (oracle/backward.py), CPU only.

The gradients are checked against things other than themselves:
* central finite differences of the C forward oracle (a separate
  implementation of the recurrence), along random directions, for every
  input, on tiny packed batches (the loss is sum(do * o) + sum(dhT * h_T));
* closed forms: with k = 0 the state only decays, o_t = (exp(G_t) o q_t)^T h0
  per channel, whose gradients are explicit sums; with beta = 0, dv = 0;
* linearity in the incoming gradients (do, dhT).
test_oracle_backward_mutants.py plants mistakes in copies of the oracle and
checks these pins catch each one.  Every pin takes the module as `B`.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as ORACLE


def _case(seed, T=6, H=2, Dk=5, Dv=4, lengths=None, h0=True):
    g = np.random.default_rng(seed)
    q = g.standard_normal((T, H, Dk))
    k = g.standard_normal((T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((T, H, Dv))
    la = -5.0 / (1.0 + np.exp(-g.standard_normal((T, H, Dk))))
    b = 1.0 / (1.0 + np.exp(-g.standard_normal((T, H))))
    N = 1 if lengths is None else len(lengths)
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)])
    h0v = g.standard_normal((N, H, Dk, Dv)) * 0.5 if h0 else None
    do = g.standard_normal((T, H, Dv))
    dhT = g.standard_normal((N, H, Dk, Dv))
    return dict(q=q, k=k, v=v, log_alpha=la, beta=b, h0=h0v, cu=cu, do=do, dhT=dhT)


def _loss(c, **over):
    x = dict(c)
    x.update(over)
    o, hT = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], h0=x["h0"],
                       cu_seqlens=x["cu"])
    return float(np.sum(c["do"] * o) + np.sum(c["dhT"] * hT))


def _grads(B, c):
    return dict(zip(("q", "k", "v", "log_alpha", "beta", "h0"),
                    B.bwd(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"], c["do"],
                          dhT=c["dhT"], h0=c["h0"], cu_seqlens=c["cu"])))


def pin_finite_differences(B):
    for seed, kw in ((1, {}), (2, dict(T=9, lengths=[4, 0, 5])), (3, dict(T=5, h0=False)),
                     (4, dict(T=8, lengths=[1, 1, 6], Dk=4, Dv=6))):
        c = _case(seed, **kw)
        gr = _grads(B, c)
        rng = np.random.default_rng(100 + seed)
        for name in ("q", "k", "v", "log_alpha", "beta", "h0"):
            if c[name] is None:
                continue
            for _ in range(3):
                d = rng.standard_normal(c[name].shape)
                eps = 1e-6
                fd = (_loss(c, **{name: c[name] + eps * d}) -
                      _loss(c, **{name: c[name] - eps * d})) / (2 * eps)
                an = float(np.sum(gr[name] * d))
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, seed, fd, an)


def pin_pure_decay_closed_form(B):
    """k = 0: o_t[j] = sum_i q_t[i] exp(G_t[i]) h0[i, j] with G_t the running
    sum of log alpha, h_T = Diag(exp(G_T)) h0."""
    c = _case(5, T=7, H=1)
    c["k"] = np.zeros_like(c["k"])
    gr = _grads(B, c)
    q, la, h0, do, dhT = c["q"][:, 0], c["log_alpha"][:, 0], c["h0"][0, 0], c["do"][:, 0], \
        c["dhT"][0, 0]
    G = np.cumsum(la, axis=0)                    # [T, Dk]
    E = np.exp(G)
    w = h0 @ do.T                                # w[i, t] = sum_j h0[i, j] do_t[j]
    dq = (E * w.T)                               # dq_t[i] = exp(G_t[i]) w[i, t]
    assert np.allclose(gr["q"][:, 0], dq, rtol=1e-12, atol=1e-12)
    # d/d la_s[i] = sum_{t >= s} q_t[i] E_t[i] w[i, t] + E_T[i] sum_j dhT[i, j] h0[i, j]
    per_t = q * E * w.T
    tail = E[-1] * np.sum(dhT * h0, axis=1)
    dla = np.cumsum(per_t[::-1], axis=0)[::-1] + tail[None, :]
    assert np.allclose(gr["log_alpha"][:, 0], dla, rtol=1e-12, atol=1e-12)
    # dh0[i, j] = sum_t q_t[i] E_t[i] do_t[j] + E_T[i] dhT[i, j]
    dh0 = (q * E).T @ do + E[-1][:, None] * dhT
    assert np.allclose(gr["h0"][0, 0], dh0, rtol=1e-12, atol=1e-12)
    assert not gr["v"].any() or np.allclose(gr["v"], 0)   # nothing is written when k = 0


def pin_no_write_no_value_gradient(B):
    c = _case(6, T=6, H=2)
    c["beta"] = np.zeros_like(c["beta"])
    gr = _grads(B, c)
    assert np.array_equal(gr["v"], np.zeros_like(c["v"]))


def pin_linear_in_incoming_gradients(B):
    c = _case(7, T=5, H=2, lengths=[2, 3])
    g1 = _grads(B, c)
    c2 = dict(c)
    c2["do"], c2["dhT"] = 2.0 * c["do"], 2.0 * c["dhT"]
    g2 = _grads(B, c2)
    c3 = dict(c)
    c3["do"], c3["dhT"] = np.zeros_like(c["do"]), np.zeros_like(c["dhT"])
    g3 = _grads(B, c3)
    for n in g1:
        assert np.allclose(g2[n], 2.0 * g1[n], rtol=1e-12, atol=1e-14), n
        assert not np.any(g3[n]), n


PINS = [pin_finite_differences, pin_pure_decay_closed_form, pin_no_write_no_value_gradient,
        pin_linear_in_incoming_gradients]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(ORACLE)
