"""Backward pass (kda_chunk_bwd) against the float64 reverse-mode oracle
(oracle/backward.py, pinned by finite differences of the forward oracle).

Loss = sum(do * o) + sum(dhT * h_T); gradients with respect to q, k, v,
log alpha, beta and h0, over packed sequences with ragged chunks.
"""
import numpy as np
import pytest
import torch

import kda_inputs
from oracle import backward as obwd
from gpu_util import TOL, case, check, need_gpu, np_

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0")


def _inputs(T, H, dtype, seed, lengths=None, h0=True, dhT=True, decay_mu=0.0):
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=seed, lengths=lengths,
                                  h0_std=0.1 if h0 else None, decay_mu=decay_mu)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed * 7 + 1)
    d["do"] = torch.randn((T, H, 128), generator=g, device="cuda").to(d["q"].dtype)
    N = d["N"]
    d["dhT"] = (torch.randn((N, H, 128, 128), generator=g, device="cuda") * 0.1) if dhT else None
    return d


def _gpu(kda, d):
    out = kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["do"],
                            h0=d["h0"], cu_seqlens=d["cu_seqlens"], dhT=d["dhT"])
    torch.cuda.synchronize()
    return out


def _oracle(d, heads=None):
    def hs(t, axis):
        if t is None:
            return None
        a = np_(t)
        return a if heads is None else np.take(a, list(heads), axis=axis)
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].cpu().numpy().astype(np.int64)
    return obwd.bwd(hs(d["q"], 1), hs(d["k"], 1), hs(d["v"], 1), hs(d["log_alpha"], 1),
                    hs(d["beta"], 1), hs(d["do"], 1), dhT=hs(d["dhT"], 1), h0=hs(d["h0"], 1),
                    cu_seqlens=cu)


BWD_CASES = [
    # dtype, T, H, lengths, decay_mu
    ("f32", 100, 2, None, 0.0),
    ("bf16", 100, 2, None, 0.0),
    ("f32", 104, 2, [37, 16, 0, 1, 50], 0.0),
    ("bf16", 104, 2, [37, 16, 0, 1, 50], 0.0),
    ("bf16", 200, 2, None, -6.0),                 # slow decay: long memory
    ("f32", 200, 2, [120, 80], -6.0),
    ("bf16", 160, 64, [40] * 4, 0.0),             # 256 chains: the whole-head recursion
]


@pytest.mark.parametrize("dtype,T,H,lengths,mu", BWD_CASES)
def test_backward_matches_oracle(dtype, T, H, lengths, mu):
    kda = need_gpu()
    case(f"backward dtype={dtype} T={T} H={H} lengths={lengths} decay_mu={mu}")
    d = _inputs(T, H, dtype, seed=31 + T + H, lengths=lengths, decay_mu=mu)
    got = _gpu(kda, d)
    heads = None if H <= 2 else (0, H - 1)
    ref = _oracle(d, heads)
    for name, gv, r in zip(NAMES, got, ref):
        x = np_(gv)
        if heads is not None:
            x = np.take(x, list(heads), axis=1)
        check(name, x, r, TOL[dtype])


def test_backward_without_h0_and_dhT():
    kda = need_gpu()
    case("backward no h0, no dhT, bf16 T=64 H=2")
    d = _inputs(64, 2, "bf16", seed=5, h0=False, dhT=False)
    got = _gpu(kda, d)
    ref = _oracle(d)
    for name, gv, r in zip(NAMES, got, ref):
        check(name, np_(gv), r, TOL["bf16"])


def test_backward_full_size_sampled_heads():
    """The 4096-token, 96-head workload in bf16, checked on sampled heads."""
    kda = need_gpu()
    T, H = 4096, 96
    case(f"backward full size T={T} H={H}")
    d = _inputs(T, H, "bf16", seed=4097, h0=False, dhT=False)
    got = _gpu(kda, d)
    heads = (0, 95)
    ref = _oracle(d, heads)
    for name, gv, r in zip(NAMES, got, ref):
        check(f"{name} heads {heads}", np.take(np_(gv), list(heads), axis=1), r, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_decay_at_the_bound(dtype):
    """log alpha = -5 on every channel: a 16-token chunk spans e^-80, the
    largest reciprocal factor the chunk form meets."""
    kda = need_gpu()
    case(f"backward decay at the bound dtype={dtype}")
    d = _inputs(80, 2, dtype, seed=91)
    d["log_alpha"].fill_(-5.0)
    got = _gpu(kda, d)
    ref = _oracle(d)
    for name, gv, r in zip(NAMES, got, ref):
        check(name, np_(gv), r, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_no_decay_full_writes(dtype):
    """log alpha = 0 and beta = 1: the plain delta rule with full overwrites."""
    kda = need_gpu()
    case(f"backward no decay, beta = 1, dtype={dtype}")
    d = _inputs(64, 2, dtype, seed=92)
    d["log_alpha"].zero_()
    d["beta"].fill_(1.0)
    got = _gpu(kda, d)
    ref = _oracle(d)
    for name, gv, r in zip(NAMES, got, ref):
        check(name, np_(gv), r, TOL[dtype])


def test_backward_single_token_and_empty():
    kda = need_gpu()
    case("backward T=1 H=1, and all-empty sequences")
    d = _inputs(1, 1, "bf16", seed=93)
    got = _gpu(kda, d)
    ref = _oracle(d)
    for name, gv, r in zip(NAMES, got, ref):
        check(name, np_(gv), r, TOL["bf16"])
    e = _inputs(0, 2, "bf16", seed=94, lengths=[0, 0])
    got = _gpu(kda, e)
    # no tokens: dh0 is dhT itself
    assert torch.equal(got[5], e["dhT"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_bitwise_reproducible_over_any_workspace(dtype):
    """Gradients are a deterministic function of the inputs: bit for bit the
    same on every run (no floating-point atomics in any reduction), and
    whatever the workspace held before the call (zeros, all-ones bytes --
    NaN in both table dtypes -- or random bytes), so no table entry is read
    before this call has written it.  Packed sequences with a one-token
    last chunk, a partial one, an empty sequence and a long one."""
    kda = need_gpu()
    lengths = [17, 23, 0, 70]
    T, H = sum(lengths), 3
    case(f"backward determinism {dtype} T={T} H={H} lengths={lengths}")
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=81, lengths=lengths,
                                  h0_std=0.1)
    g = torch.Generator(device="cuda").manual_seed(81)
    do = torch.randn((T, H, 128), generator=g, device="cuda").to(d["q"].dtype)
    dhT = torch.randn((len(lengths), H, 128, 128), generator=g, device="cuda") * 0.1
    nbytes = kda.kda_chunk_bwd_workspace_size(T, len(lengths), H,
                                              dtype=kda.KDA_BF16 if dtype == "bf16" else kda.KDA_F32)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    runs = []
    for fill in ("zeros", "ones", "random"):
        if fill == "zeros":
            ws.zero_()
        elif fill == "ones":
            ws.fill_(0xFF)
        else:
            ws.copy_(torch.randint(0, 256, (nbytes,), generator=g, device="cuda",
                                   dtype=torch.int32).to(torch.uint8))
        runs.append(kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], do,
                                      h0=d["h0"], cu_seqlens=d["cu_seqlens"], dhT=dhT,
                                      workspace=ws))
        torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0")
    for r in runs[1:]:
        for name, a, b in zip(names, r, runs[0]):
            assert torch.isfinite(a.float()).all(), f"{name}: non-finite"
            assert torch.equal(a, b), f"{name} differs between runs"
