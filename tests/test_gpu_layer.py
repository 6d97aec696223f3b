"""The prologue and epilogue of a KDA layer (kda_prologue, kda_epilogue)
against the fp64 oracle (oracle/layer.py), element by element.

Prologue: q, k, v = Swish(width-4 causal depthwise conv), q and k
L2-normalised per head, log alpha = -5 sigmoid(a + bias), beta = sigmoid(b),
and the convolution history of every sequence; epilogue: head RMSNorm times
the sigmoid output gate ("From GPT-2 to Kimi K3", ch. 6; "An infra-oriented
diagram of Kimi K3", Kimi Delta Attention card).
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from oracle import layer as olayer
from gpu_util import TOL, case, check, need_gpu, np_

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_alpha", "beta")


def _gpu_prologue(kda, d, conv_state="from_inputs", store_state=True):
    cs = d["conv_state"] if conv_state == "from_inputs" else conv_state
    out = kda.kda_prologue(d["xq"], d["xk"], d["xv"], d["a_raw"], d["b_raw"], d["conv_w"],
                           d["a_bias"], cu_seqlens=d["cu_seqlens"], conv_state=cs,
                           store_state=store_state)
    torch.cuda.synchronize()
    return out


def _oracle_prologue(d, heads=None):
    """fp64 oracle on the same input values (optionally a subset of heads:
    every step is per head, so a head slice is exact)."""
    sel = slice(None) if heads is None else list(heads)

    def hs(t, axis):
        a = np_(t)
        return a if heads is None else np.take(a, sel, axis=axis)

    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].cpu().numpy().astype(np.int64)
    cs = None if d["conv_state"] is None else hs(d["conv_state"], 3)
    return olayer.prologue(hs(d["xq"], 1), hs(d["xk"], 1), hs(d["xv"], 1), hs(d["a_raw"], 1),
                           hs(d["b_raw"], 1), hs(d["conv_w"], 1), hs(d["a_bias"], 0),
                           cu_seqlens=cu, conv_state=cs)


PROLOGUE_CASES = [
    # dtype, T, H, lengths, cached history
    ("bf16", 300, 3, [100, 3, 0, 197], True),
    ("f32", 300, 3, [100, 3, 0, 197], True),
    ("bf16", 1000, 5, None, False),
    ("bf16", 64, 4, [1] * 64, True),                 # a decode step of 64 requests
    ("f32", 64, 4, [1] * 64, True),
    ("bf16", 77, 2, [1, 2, 3, 4, 0, 67], True),      # sequences shorter than the window
    ("bf16", 4100, 6, [4000, 100], False),           # several token blocks per wave row
    ("bf16", 33, 1, [10, 23], True),                 # one head: three dead rows per wave
    ("f32", 1, 1, None, True),                       # one token
]


@pytest.mark.parametrize("dtype,T,H,lengths,hist", PROLOGUE_CASES)
def test_prologue_matches_oracle(dtype, T, H, lengths, hist):
    kda = need_gpu()
    case(f"prologue dtype={dtype} T={T} H={H} lengths={lengths} history={hist}")
    d = kda_inputs.layer_inputs(T, H, dtype=dtype, device="cuda", seed=17 + T + H,
                                lengths=lengths, conv_state=hist)
    got = _gpu_prologue(kda, d)
    ref = _oracle_prologue(d)
    for name, g, r in zip(NAMES, got[:5], ref[:5]):
        check(name, np_(g), r, TOL[dtype])
    # the history is a copy of inputs: exact
    assert np.array_equal(np_(got[5]), ref[5]), "convolution history differs"


def test_prologue_full_size_sampled_heads():
    """The 4096-token, 96-head workload in bf16, checked on sampled heads."""
    kda = need_gpu()
    T, H = 4096, 96
    case(f"prologue full size T={T} H={H}")
    d = kda_inputs.layer_inputs(T, H, dtype="bf16", device="cuda", seed=4096)
    got = _gpu_prologue(kda, d)
    heads = [0, 37, 95]
    ref = _oracle_prologue(d, heads)
    for name, g, r in zip(NAMES, got[:5], ref[:5]):
        check(f"{name} heads {heads}", np_(g)[:, heads], r, TOL["bf16"])
    assert np.array_equal(np_(got[5])[:, :, :, heads], ref[5])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prologue_split_with_history_is_bitwise_the_whole(dtype):
    """Running a sequence in pieces, handing the history on, reproduces the
    one-shot prologue exactly (the same values enter every window)."""
    kda = need_gpu()
    T, H = 260, 3
    case(f"prologue split dtype={dtype} T={T} H={H}")
    d = kda_inputs.layer_inputs(T, H, dtype=dtype, device="cuda", seed=99, conv_state=True)
    whole = _gpu_prologue(kda, d)
    cs = d["conv_state"]
    parts = []
    for a, b in ((0, 1), (1, 3), (3, 100), (100, 101), (101, T)):
        sub = dict(d)
        for x in ("xq", "xk", "xv", "a_raw", "b_raw"):
            sub[x] = d[x][a:b].contiguous()
        out = _gpu_prologue(kda, sub, conv_state=cs)
        parts.append(out)
        cs = out[5]
    for i, name in enumerate(NAMES):
        cat = torch.cat([p[i] for p in parts])
        assert torch.equal(cat, whole[i]), f"{name} differs when split"
    assert torch.equal(cs, whole[5])


def test_prologue_all_empty_carries_history():
    kda = need_gpu()
    case("prologue T=0 with history")
    d = kda_inputs.layer_inputs(0, 2, dtype="bf16", device="cuda", seed=3, lengths=[0, 0, 0],
                                conv_state=True)
    got = _gpu_prologue(kda, d)
    assert torch.equal(got[5], d["conv_state"])
    d["conv_state"] = None
    got = _gpu_prologue(kda, d)
    assert not got[5].any()


EPILOGUE_CASES = [("bf16", 500, 3), ("f32", 500, 3), ("bf16", 4096, 96), ("f32", 1, 1)]


@pytest.mark.parametrize("dtype,T,H", EPILOGUE_CASES)
def test_epilogue_matches_oracle(dtype, T, H):
    kda = need_gpu()
    case(f"epilogue dtype={dtype} T={T} H={H}")
    d = kda_inputs.layer_inputs(T, H, dtype=dtype, device="cuda", seed=7 + T)
    y = kda.kda_epilogue(d["o"], d["g"], d["norm_w"])
    torch.cuda.synchronize()
    if H > 8:   # sampled heads at full size
        heads = [0, H // 2, H - 1]
        ref = olayer.epilogue(np_(d["o"])[:, heads], np_(d["g"])[:, heads],
                              np_(d["norm_w"])[heads])
        check(f"y heads {heads}", np_(y)[:, heads], ref, TOL[dtype])
    else:
        ref = olayer.epilogue(np_(d["o"]), np_(d["g"]), np_(d["norm_w"]))
        check("y", np_(y), ref, TOL[dtype])
    # in place over o gives the same bits
    o2 = d["o"].clone()
    kda.kda_epilogue(o2, d["g"], d["norm_w"], y=o2)
    torch.cuda.synchronize()
    assert torch.equal(o2, y)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layer_chain_matches_oracle_chain(dtype):
    """prologue -> chunkwise core -> epilogue on the GPU equals the same
    chain of oracles (the GPU rounds its intermediates to the I/O dtype)."""
    kda = need_gpu()
    T, H, lengths = 400, 2, [150, 250]
    case(f"layer chain dtype={dtype} T={T} H={H}")
    d = kda_inputs.layer_inputs(T, H, dtype=dtype, device="cuda", seed=400, lengths=lengths)
    q, k, v, la, beta, _ = _gpu_prologue(kda, d, store_state=False)
    o, _ = kda.kda_chunk_fwd(q, k, v, la, beta, cu_seqlens=d["cu_seqlens"])
    y = kda.kda_epilogue(o, d["g"], d["norm_w"])
    torch.cuda.synchronize()
    rq, rk, rv, rla, rb, _ = _oracle_prologue(d)
    cu = d["cu_seqlens"].cpu().numpy().astype(np.int64)
    ro, _ = oracle.fwd(rq, rk, rv, rla, rb, cu_seqlens=cu)
    ry = olayer.epilogue(ro, np_(d["g"]), np_(d["norm_w"]))
    check("y (whole layer)", np_(y), ry, TOL[dtype])
