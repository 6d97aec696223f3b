"""Pins of the CPU oracle to what the pages and the mathematics fix.

Every test here checks the oracle (oracle/kda_oracle.c) against something
other than itself: values printed on the pages (tests/golden/), closed
forms, the explicit-matrix evaluation of the published equation
(tests/brute.py), algebraic invariants and special cases that reduce to
simpler, separately written rules.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from brute import affine_segment, transition, unrolled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rand_inputs(rng, T, H, Dk, Dv, unit=True, g_scale=1.0):
    q = rng.standard_normal((T, H, Dk))
    k = rng.standard_normal((T, H, Dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, Dv))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((T, H, Dk)))) * g_scale
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, b


def nerr(x, ref):
    """Normwise error max|x - ref| / max|ref|."""
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300))


# ---------------------------------------------------------------- golden ----

def test_golden_overwrite_2d():
    """beta = 1 with a unit key overwrites the prediction exactly
    ("From GPT-2 to Kimi K3", ch. 3, "A complete overwrite")."""
    g = golden("overwrite_2d.json")
    S0 = np.array(g["S0"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    la = np.array(g["log_alpha"])[None, None]
    b = np.array([[g["beta"]]])
    assert np.allclose(S0[0, 0].T @ k[0, 0], g["prediction_before"])
    o, S1 = oracle.fwd(k, k, v, la, b, h0=S0)            # read with q = k
    row = int(np.argmax(np.abs(g["k"])))
    assert np.array_equal(S1[0, 0][row], np.array(g["row_after"]))
    assert np.array_equal(o[0, 0], np.array(g["read_after"]))
    assert np.array_equal(S1[0, 0].T @ k[0, 0], np.array(g["read_after"]))


@pytest.mark.parametrize("case", golden("half_life.json")["cases"])
def test_golden_half_life(case):
    """With beta = 0 and constant retention alpha, the state halves after the
    page's half-life ("From GPT-2 to Kimi K3", ch. 4)."""
    a, n_half = case["alpha"], case["half_life_tokens"]
    T, d = n_half + 1, 4
    rng = np.random.default_rng(7)
    S0 = rng.standard_normal((1, 1, d, d))
    z = np.zeros((T, 1, d))
    la = np.full((T, 1, d), math.log(a))
    b = np.zeros((T, 1))
    # the state after t tokens is read back through o_t = S_t^T e_i for each i
    ratios = []
    for t in (n_half - 1, n_half):
        _, St = oracle.fwd(z[:t], z[:t], z[:t], la[:t], b[:t], h0=S0)
        ratios.append(float(np.abs(St).max() / np.abs(S0).max()))
    assert ratios[0] > 0.5 >= ratios[1], ratios


def test_golden_decay_bound():
    """e^-5 ~ 0.0067 is the retention infimum; a 16-token tile at the bound
    decays by e^-80, whose reciprocal is below the bf16 maximum
    ("From GPT-2 to Kimi K3", ch. 5; KDA card of the infra diagram)."""
    g = golden("decay_bound.json")
    assert round(math.exp(g["log_decay_min"]), g["alpha_infimum_digits"]) == \
        g["alpha_infimum_approx"]
    cum = g["tile_tokens"] * g["log_decay_min"]
    assert cum == g["tile_cumulative_log_decay_min"]
    bf16_max = float(torch.finfo(torch.bfloat16).max)
    f16_max = float(torch.finfo(torch.float16).max)
    assert math.exp(-cum) < bf16_max          # representable in bf16
    assert math.exp(-cum) > f16_max           # ... but not in fp16
    # the oracle at the bound: beta = 0, 16 tokens, log alpha = -5 everywhere
    T, d = g["tile_tokens"], 8
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((1, 1, d, d))
    z = np.zeros((T, 1, d))
    _, St = oracle.fwd(z, z, z, np.full((T, 1, d), -5.0), np.zeros((T, 1)), h0=S0)
    assert nerr(St, S0 * math.exp(cum)) < 1e-12


# ------------------------------------------------------- closed forms -------

def test_overwrite_unit_key_any_decay():
    """beta = 1 and ||k|| = 1 make S_t^T k_t = v_t exactly, whatever the decay
    and the previous state (ch. 3 "A complete overwrite", with the unit-key
    condition stated there)."""
    rng = np.random.default_rng(11)
    T, H, D = 9, 3, 32
    q, k, v, g, b = rand_inputs(rng, T, H, D, D)
    b[:] = 1.0
    h0 = rng.standard_normal((1, H, D, D))
    # check after every token by running prefixes
    for t in range(1, T + 1):
        _, St = oracle.fwd(q[:t], k[:t], v[:t], g[:t], b[:t], h0=h0)
        for h in range(H):
            assert np.abs(St[0, h].T @ k[t - 1, h] - v[t - 1, h]).max() < 1e-12


def test_beta0_alpha1_state_unchanged():
    """beta = 0 and alpha = 1 leave S untouched, so o_t = h0^T q_t
    (ch. 4: alpha = 1 means no decay; beta = 0 writes nothing)."""
    rng = np.random.default_rng(12)
    T, H, D = 20, 2, 16
    q, k, v, g, b = rand_inputs(rng, T, H, D, D)
    h0 = rng.standard_normal((1, H, D, D))
    o, hT = oracle.fwd(q, k, v, np.zeros_like(g), np.zeros_like(b), h0=h0)
    assert np.array_equal(hT, h0)
    ref = np.einsum("hij,thi->thj", h0[0], q)
    assert nerr(o, ref) < 1e-13
    # constant q gives constant read-out
    qc = np.broadcast_to(q[:1], q.shape)
    oc, _ = oracle.fwd(qc, k, v, np.zeros_like(g), np.zeros_like(b), h0=h0)
    assert np.allclose(oc, oc[:1], rtol=0, atol=1e-14)


def test_beta0_channelwise_decay_closed_form():
    """beta = 0: S_t = Diag(exp(sum_s log alpha_s)) S_0 -- each ROW (key
    channel) decays by its own running product ("Kimi K3 Architecture
    Explained", Step 3: Diag(alpha) scales each row; the running-product
    reading of the token-1 labels)."""
    rng = np.random.default_rng(13)
    T, H, Dk, Dv = 37, 2, 12, 5
    q, k, v, g, b = rand_inputs(rng, T, H, Dk, Dv)
    h0 = rng.standard_normal((1, H, Dk, Dv))
    _, hT = oracle.fwd(q, k, v, g, np.zeros_like(b), h0=h0)
    scale = np.exp(g.sum(axis=0))                  # [H, Dk]
    ref = h0[0] * scale[:, :, None]
    assert nerr(hT[0], ref) < 1e-12


def test_delta_rule_special_case():
    """log alpha = 0 reduces KDA to the delta rule
    S_t = (I - beta k k^T) S_{t-1} + beta k v^T ("Kimi K3 Architecture
    Explained", Step 2, the combined delta-rule equation), evaluated here as
    recall / compare / correct with explicit vectors."""
    rng = np.random.default_rng(14)
    T, H, Dk, Dv = 25, 2, 10, 7
    q, k, v, g, b = rand_inputs(rng, T, H, Dk, Dv, unit=False)
    h0 = rng.standard_normal((1, H, Dk, Dv))
    o, hT = oracle.fwd(q, k, v, np.zeros_like(g), b, h0=h0)
    for h in range(H):
        S = h0[0, h].copy()
        for t in range(T):
            vhat = S.T @ k[t, h]                       # recall
            delta = v[t, h] - vhat                     # compare
            S = S + b[t, h] * np.outer(k[t, h], delta)  # correct
            assert nerr(o[t, h], S.T @ q[t, h]) < 1e-12
        assert nerr(hT[0, h], S) < 1e-12


def test_gated_deltanet_special_case():
    """alpha equal across channels reduces KDA to Gated DeltaNet,
    S_t = alpha_t (I - beta k k^T) S_{t-1} + beta k v^T (the blog's
    scalar-gate form; for a scalar the order of alpha and the erase factor
    does not matter)."""
    rng = np.random.default_rng(15)
    T, H, Dk, Dv = 25, 2, 9, 6
    q, k, v, g, b = rand_inputs(rng, T, H, Dk, Dv)
    gs = np.broadcast_to(g[:, :, :1], g.shape).copy()   # one alpha per token
    h0 = rng.standard_normal((1, H, Dk, Dv))
    o, hT = oracle.fwd(q, k, v, gs, b, h0=h0)
    for h in range(H):
        S = h0[0, h].copy()
        for t in range(T):
            a = math.exp(gs[t, h, 0])
            S = a * (np.eye(Dk) - b[t, h] * np.outer(k[t, h], k[t, h])) @ S \
                + b[t, h] * np.outer(k[t, h], v[t, h])
            assert nerr(o[t, h], S.T @ q[t, h]) < 1e-12
        assert nerr(hT[0, h], S) < 1e-12


def test_one_hot_keys_row_ema():
    """k_t = e_{i_t}: row i_t becomes (1 - beta) alpha_{i_t} row + beta v_t and
    every other row only decays -- rows are key channels."""
    rng = np.random.default_rng(16)
    T, H, Dk, Dv = 30, 1, 6, 4
    q, _, v, g, b = rand_inputs(rng, T, H, Dk, Dv)
    idx = rng.integers(0, Dk, size=T)
    k = np.zeros((T, H, Dk))
    k[np.arange(T), 0, idx] = 1.0
    h0 = rng.standard_normal((1, H, Dk, Dv))
    _, hT = oracle.fwd(q, k, v, g, b, h0=h0)
    S = h0[0, 0].copy()
    for t in range(T):
        a = np.exp(g[t, 0])
        S = S * a[:, None]
        i = idx[t]
        S[i] = (1.0 - b[t, 0]) * S[i] + b[t, 0] * v[t, 0]
    assert nerr(hT[0, 0], S) < 1e-13


# --------------------------------------------------------- brute force ------

@pytest.mark.parametrize("Dk,Dv,T", [(5, 3, 8), (3, 7, 6), (16, 16, 8), (128, 128, 4)])
def test_brute_force_unrolled_products(Dk, Dv, T):
    """The oracle equals the explicit-matrix unrolling of the published
    equation, M_t = (I - beta k k^T) Diag(alpha) (non-unit keys, non-square
    state, random h0)."""
    rng = np.random.default_rng(17 + Dk + Dv)
    q, k, v, g, b = rand_inputs(rng, T, 2, Dk, Dv, unit=False)
    k *= 0.5
    h0 = rng.standard_normal((1, 2, Dk, Dv))
    o, hT = oracle.fwd(q, k, v, g, b, h0=h0)
    for h in range(2):
        ob, Sb = unrolled(q[:, h], k[:, h], v[:, h], g[:, h], b[:, h], h0[0, h])
        assert nerr(o[:, h], ob) < 1e-11
        assert nerr(hT[0, h], Sb) < 1e-11


def test_read_after_update():
    """Token t reads the state after its own update ("From GPT-2 to Kimi K3",
    ch. 6): from a zero state, o_1 = beta (k.q) v, not zero."""
    rng = np.random.default_rng(18)
    q, k, v, g, b = rand_inputs(rng, 1, 1, 8, 8)
    o, _ = oracle.fwd(q, k, v, g, b)
    ref = b[0, 0] * float(k[0, 0] @ q[0, 0]) * v[0, 0]
    assert nerr(o[0, 0], ref) < 1e-14


# ------------------------------------------------------------ invariants ----

def test_affine_segment_composition():
    """A segment acts on its incoming state as an affine map S -> A S + B;
    two segments compose associatively, (A2 A1, A2 B1 + B2)
    ("From GPT-2 to Kimi K3", ch. 6, "Context parallelism is not simple
    summation")."""
    rng = np.random.default_rng(19)
    T, Dk, Dv, split = 12, 6, 4, 5
    # slow decay so that the incoming state's part is not negligible
    q, k, v, g, b = rand_inputs(rng, T, 1, Dk, Dv, g_scale=0.05)
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    _, hT = oracle.fwd(q, k, v, g, b, h0=S0)
    A1, B1 = affine_segment(k[:split, 0], g[:split, 0], b[:split, 0], v[:split, 0])
    A2, B2 = affine_segment(k[split:, 0], g[split:, 0], b[split:, 0], v[split:, 0])
    A, B = A2 @ A1, A2 @ B1 + B2
    assert nerr(hT[0, 0], A @ S0[0, 0] + B) < 1e-12
    # the oracle itself is affine in h0: f(x S + y R) - f(0) is linear
    R = rng.standard_normal(S0.shape)
    _, f0 = oracle.fwd(q, k, v, g, b)
    _, fS = oracle.fwd(q, k, v, g, b, h0=S0)
    _, fR = oracle.fwd(q, k, v, g, b, h0=R)
    _, fm = oracle.fwd(q, k, v, g, b, h0=2.0 * S0 - 3.0 * R)
    assert nerr(fm - f0, 2.0 * (fS - f0) - 3.0 * (fR - f0)) < 1e-12
    assert nerr(f0[0, 0], B2 + A2 @ B1) < 1e-12


def test_contraction_bound():
    """With a unit key, beta in [0, 1] and alpha in (0, 1], the erase factor
    (I - beta k k^T) Diag(alpha) cannot amplify the state:
    ||S_t||_2 <= ||S_{t-1}||_2 + beta ||v_t|| ("Kimi K3 Architecture
    Explained", "Inside a KDA Layer": unit keys keep or shrink the state)."""
    rng = np.random.default_rng(20)
    T, D = 40, 16
    q, k, v, g, b = rand_inputs(rng, T, 1, D, D)
    S = rng.standard_normal((1, 1, D, D)) * 3.0
    for t in range(T):
        assert np.linalg.norm(transition(k[t, 0], g[t, 0], b[t, 0]), 2) <= 1 + 1e-12
        _, Sn = oracle.fwd(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                           b[t:t + 1], h0=S)
        lhs = np.linalg.norm(Sn[0, 0], 2)
        rhs = np.linalg.norm(S[0, 0], 2) + b[t, 0] * np.linalg.norm(v[t, 0])
        assert lhs <= rhs + 1e-12
        S = Sn


def test_value_column_independence():
    """Running on a subset of value columns (v and the state) reproduces
    those columns exactly -- what makes splitting d_v legal."""
    rng = np.random.default_rng(21)
    T, H, Dk, Dv = 33, 2, 16, 12
    q, k, v, g, b = rand_inputs(rng, T, H, Dk, Dv)
    h0 = rng.standard_normal((1, H, Dk, Dv))
    o, hT = oracle.fwd(q, k, v, g, b, h0=h0)
    cols = np.array([1, 4, 5, 11])
    os_, hs = oracle.fwd(q, k, v[:, :, cols], g, b, h0=h0[:, :, :, cols])
    assert np.array_equal(os_, o[:, :, cols])
    assert np.array_equal(hs, hT[:, :, :, cols])
    # and the oracle's own column blocking changes nothing
    ob, hb = oracle.fwd(q, k, v, g, b, h0=h0, dv_block=5, nthreads=3)
    assert np.array_equal(ob, o) and np.array_equal(hb, hT)


def test_resume_equals_single_pass():
    """fwd(T1 + T2) = fwd(T2, h0 = h_T(T1)): the state is the checkpoint."""
    rng = np.random.default_rng(22)
    T, H, D, T1 = 50, 3, 16, 21
    q, k, v, g, b = rand_inputs(rng, T, H, D, D)
    h0 = rng.standard_normal((1, H, D, D))
    o, hT = oracle.fwd(q, k, v, g, b, h0=h0)
    o1, h1 = oracle.fwd(q[:T1], k[:T1], v[:T1], g[:T1], b[:T1], h0=h0)
    o2, h2 = oracle.fwd(q[T1:], k[T1:], v[T1:], g[T1:], b[T1:], h0=h1)
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(h2, hT)


def test_varlen_is_independent_runs():
    """Packed documents with cumulative offsets behave as separate runs, each
    from its own h0 ("An infra-oriented diagram of Kimi K3": packed tokens,
    boundaries preserved by cumulative sequence offsets); an empty document
    returns its h0."""
    rng = np.random.default_rng(23)
    lens = [7, 0, 1, 19, 16]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, D = int(cu[-1]), 2, 8
    q, k, v, g, b = rand_inputs(rng, T, H, D, D)
    h0 = rng.standard_normal((len(lens), H, D, D))
    o, hT = oracle.fwd(q, k, v, g, b, h0=h0, cu_seqlens=cu)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, hn = oracle.fwd(q[s:e], k[s:e], v[s:e], g[s:e], b[s:e], h0=h0[n:n + 1])
        assert np.array_equal(o[s:e], on)
        assert np.array_equal(hT[n], hn[0])
    assert np.array_equal(hT[1], h0[1])


def test_decode_equals_one_token_prefill():
    """The fused-recurrent single-token step is the chunk path with T = 1
    ("From GPT-2 to Kimi K3", ch. 6, the mode rule)."""
    rng = np.random.default_rng(24)
    B, H, D = 5, 3, 16
    q, k, v, g, b = rand_inputs(rng, B, H, D, D)
    S = rng.standard_normal((B, H, D, D))
    od, Sd = oracle.decode(q, k, v, g, b, S)
    cu = np.arange(B + 1)
    of, hf = oracle.fwd(q, k, v, g, b, h0=S, cu_seqlens=cu)
    assert np.array_equal(od, of)
    assert np.array_equal(Sd, hf)


def test_fp32_oracle_close_to_fp64():
    """The float build (the timed CPU baseline) stays within 1e-5 normwise of
    the double build on a K3-shaped head."""
    rng = np.random.default_rng(25)
    T, H, D = 256, 2, 128
    q, k, v, g, b = rand_inputs(rng, T, H, D, D)
    h0 = 0.02 * rng.standard_normal((1, H, D, D))
    o64, h64 = oracle.fwd(q, k, v, g, b, h0=h0)
    o32, h32 = oracle.fwd(q, k, v, g, b, h0=h0, precision="f32")
    assert nerr(o32, o64) < 1e-5
    assert nerr(h32, h64) < 1e-5


def test_rejects_bad_offsets():
    rng = np.random.default_rng(26)
    q, k, v, g, b = rand_inputs(rng, 4, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, g, b, cu_seqlens=[0, 3, 2, 4])
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, g, b, cu_seqlens=[0, 3])
