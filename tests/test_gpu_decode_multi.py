"""kda_decode_multi: up to K recurrent steps per sequence in one pass over
its state (speculative verify and replay), against the fp64 oracle.

Token t of sequence b must give exactly what the oracle's recurrence gives
after t + 1 tokens from the cached state; a verify pass (update_state off)
must leave the cached state bit-identical, and tokens past a sequence's
accepted count must neither write outputs nor move the state ("From GPT-2 to
Kimi K3, from first principles": "Speculative decoding cannot naively roll
KDA back").
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from gpu_util import TOL, case, check, need_gpu, np_

pytestmark = pytest.mark.gpu


def _window_inputs(B, K, H, dtype, seed):
    """B sequences of K tokens each, [B, K, H, ...] views of packed tokens,
    plus cached states."""
    d = kda_inputs.prefill_inputs(B * K, H, dtype=dtype, device="cuda", seed=seed,
                                  lengths=[K] * B, h0_std=0.05, decay_mu=-4.0)
    w = {x: d[x].view(B, K, *d[x].shape[1:]) for x in ("q", "k", "v", "log_alpha", "beta")}
    return d, w


def _oracle_window(d, B, K, n, b):
    """fp64 oracle outputs and final state of sequence b over its first n tokens."""
    sl = slice(b * K, b * K + n)
    return oracle.fwd(np_(d["q"][sl]), np_(d["k"][sl]), np_(d["v"][sl]),
                      np_(d["log_alpha"][sl]), np_(d["beta"][sl]), h0=np_(d["h0"])[b:b + 1])


MULTI = [
    # dtype, B, K, H, n_tok (None = K), update_state
    ("bf16", 8, 7, 3, [7, 4, 0, 1, 7, 3, 2, 5], True),     # odd H: blocks span sequences
    ("bf16", 8, 7, 3, None, False),                          # verify pass
    ("f32", 5, 4, 2, None, True),
    ("f32", 6, 16, 2, [16, 9, 1, 0, 12, 15], True),
    ("bf16", 3, 1, 96, None, True),                          # K = 1 at the K3 width
    ("bf16", 4, 20, 3, [20, 17, 8, 9], True),                # three blocks of staged tokens
]


@pytest.mark.parametrize("dtype,B,K,H,n_tok,update", MULTI)
def test_decode_multi_matches_oracle(dtype, B, K, H, n_tok, update):
    kda = need_gpu()
    case(f"decode_multi dtype={dtype} B={B} K={K} H={H} n_tok={n_tok} update={update}")
    d, w = _window_inputs(B, K, H, dtype, seed=300 + B + K + H)
    S = d["h0"].clone()
    S_before = S.clone()
    nt = None if n_tok is None else torch.tensor(n_tok, dtype=torch.int32, device="cuda")
    sentinel = 1024.0  # exact in bf16 and fp32
    o = torch.full((B, K, H, 128), sentinel, dtype=w["q"].dtype, device="cuda")
    kda.kda_decode_multi(w["q"], w["k"], w["v"], w["log_alpha"], w["beta"], S, nt,
                         update_state=update, o=o)
    torch.cuda.synchronize()
    counts = [K] * B if n_tok is None else n_tok
    got_o, got_S = np_(o), np_(S)
    for b in range(B):
        n = counts[b]
        if n:
            ro, rh = _oracle_window(d, B, K, n, b)
            check(f"o of sequence {b} ({n} tokens)", got_o[b, :n], ro, TOL[dtype])
            if update:
                check(f"S of sequence {b}", got_S[b], rh[0], TOL[dtype])
        assert np.all(got_o[b, n:] == sentinel), f"rows past n_tok of sequence {b} written"
        if not update or n == 0:
            assert torch.equal(S[b], S_before[b]), f"state of sequence {b} moved"


def test_decode_multi_one_token_equals_decode_step():
    """K = 1 is one decode step: the two kernels sum the state's columns in a
    different order (the multi-token kernel keeps them inside a wavefront),
    so they agree to rounding, not bit for bit."""
    kda = need_gpu()
    B, H = 16, 96
    case(f"decode_multi K=1 vs decode_step B={B} H={H}")
    dd = kda_inputs.decode_inputs(B, H, dtype="bf16", device="cuda", seed=77)
    S1, S2 = dd["S"].clone(), dd["S"].clone()
    o1 = kda.kda_decode_step(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], S1)
    o2 = kda.kda_decode_multi(*[dd[x].unsqueeze(1) for x in ("q", "k", "v", "log_alpha",
                                                              "beta")], S2)
    torch.cuda.synchronize()
    check("o: multi-token K=1 vs decode step", np_(o2[:, 0]), np_(o1).astype(np.float64), 1e-2)
    check("S: multi-token K=1 vs decode step", np_(S2), np_(S1).astype(np.float64), 1e-5)


def test_decode_multi_agrees_with_the_chunk_path():
    """The same windows through the chunkwise kernel (packed sequences with h0)."""
    kda = need_gpu()
    B, K, H = 64, 7, 8
    case(f"decode_multi vs chunk path B={B} K={K} H={H}")
    d, w = _window_inputs(B, K, H, "bf16", seed=404)
    S = d["h0"].clone()
    o = kda.kda_decode_multi(w["q"], w["k"], w["v"], w["log_alpha"], w["beta"], S)
    oc, hc = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], h0=d["h0"],
                               cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    check("o: multi-token decode vs chunk", np_(o).reshape(B * K, H, 128), np_(oc), TOL["bf16"])
    check("S: multi-token decode vs chunk", np_(S), np_(hc), TOL["bf16"])


def test_decode_multi_clamps_token_counts():
    kda = need_gpu()
    B, K, H = 4, 5, 2
    case("decode_multi n_tok outside [0, K]")
    d, w = _window_inputs(B, K, H, "f32", seed=505)
    Sa, Sb = d["h0"].clone(), d["h0"].clone()
    bad = torch.tensor([-3, 99, 5, 0], dtype=torch.int32, device="cuda")
    good = torch.tensor([0, 5, 5, 0], dtype=torch.int32, device="cuda")
    oa = kda.kda_decode_multi(w["q"], w["k"], w["v"], w["log_alpha"], w["beta"], Sa, bad)
    ob = kda.kda_decode_multi(w["q"], w["k"], w["v"], w["log_alpha"], w["beta"], Sb, good)
    torch.cuda.synchronize()
    assert torch.equal(Sa, Sb)
    assert torch.equal(oa[1:3], ob[1:3])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_multi_at_the_decay_bound(dtype):
    """log alpha = -5 on every channel of every token (the bound of the input
    contract): the kernel holds the state divided by the running decay of
    each block of 8 tokens, so here that product falls to e^-40 before the
    block ends; three blocks (K = 20) check the rescaling at every block
    boundary against the oracle."""
    kda = need_gpu()
    B, K, H = 4, 20, 2
    case(f"decode_multi at the decay bound dtype={dtype} B={B} K={K} H={H}")
    d, w = _window_inputs(B, K, H, dtype, seed=777)
    d["log_alpha"].fill_(-5.0)
    S = d["h0"].clone()
    o = torch.empty((B, K, H, 128), dtype=w["q"].dtype, device="cuda")
    kda.kda_decode_multi(w["q"], w["k"], w["v"], w["log_alpha"], w["beta"], S, None,
                         update_state=True, o=o)
    torch.cuda.synchronize()
    got_o, got_S = np_(o), np_(S)
    for b in range(B):
        ro, rh = _oracle_window(d, B, K, K, b)
        check(f"o of sequence {b}", got_o[b], ro, TOL[dtype])
        check(f"S of sequence {b}", got_S[b], rh[0], TOL[dtype])
