"""HIP graph capture of the hot-path entry points.

A graph recorded around kda_chunk_fwd, kda_decode_step or kda_chunk_bwd on
static buffers, replayed after fresh inputs are copied in, gives the same
bits as the eager call on those inputs.  Every replay is checked, with eager
launches and synchronisations between replays (a recorded memset or a
launch-time host value baked into the graph would show up as a wrong replay
after the first).  The libraries set their kernels' LDS limits once per
device, so the recorded launches make no attribute calls.
"""
import pytest
import torch

import kda_inputs
from gpu_util import case, need_gpu

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_alpha", "beta")


def _capture(fn):
    """One eager call on a side stream (as torch asks before capture), then
    the recorded call; returns (graph, what the recorded call returned)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


@pytest.mark.parametrize("dtype,T,lengths", [
    ("bf16", 437, [100, 0, 37, 300]),   # pipelined kernel, ragged and empty sequences
    ("bf16", 1100, None),               # its deeper schedule (long sequences)
    ("f32", 437, [100, 0, 37, 300]),    # phase-serial kernel
])
def test_prefill_graph_replays_match_eager(dtype, T, lengths):
    kda = need_gpu()
    H = 4
    case(f"graph prefill dtype={dtype} T={T} lengths={lengths}")
    sets = [kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=s, lengths=lengths,
                                      h0_std=0.05) for s in (11, 12, 13)]
    st = {n: sets[0][n].clone() for n in NAMES + ("h0",)}
    cu = sets[0]["cu_seqlens"]
    o = torch.empty_like(st["v"])
    hT = torch.empty_like(st["h0"])

    def fn():
        return kda.kda_chunk_fwd(*[st[n] for n in NAMES], h0=st["h0"], cu_seqlens=cu, o=o, h_T=hT)

    g, _ = _capture(fn)
    for r, d in enumerate(sets):
        for n in NAMES + ("h0",):
            st[n].copy_(d[n])
        g.replay()
        torch.cuda.synchronize()
        eo, eh = kda.kda_chunk_fwd(*[d[n] for n in NAMES], h0=d["h0"], cu_seqlens=cu)
        torch.cuda.synchronize()
        print(f"  replay {r}", flush=True)
        assert torch.equal(o, eo), f"o differs on replay {r}"
        assert torch.equal(hT, eh), f"h_T differs on replay {r}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_graph_replays_match_eager(dtype):
    """The recorded step updates its state in place on every replay, as the
    eager step does on a copy of that state."""
    kda = need_gpu()
    B, H = 64, 8
    case(f"graph decode dtype={dtype} B={B} H={H}")
    sets = [kda_inputs.decode_inputs(B, H, dtype=dtype, device="cuda", seed=s) for s in (21, 22, 23)]
    st = {n: sets[0][n].clone() for n in NAMES}
    S = sets[0]["S"].clone()
    o = torch.empty_like(st["v"])

    def fn():
        return kda.kda_decode_step(*[st[n] for n in NAMES], S, o=o)

    g, _ = _capture(fn)
    S_eager = S.clone()   # the state after the warm-up call
    for r, d in enumerate(sets):
        for n in NAMES:
            st[n].copy_(d[n])
        g.replay()
        torch.cuda.synchronize()
        eo = kda.kda_decode_step(*[d[n] for n in NAMES], S_eager)
        torch.cuda.synchronize()
        print(f"  replay {r}", flush=True)
        assert torch.equal(o, eo), f"o differs on replay {r}"
        assert torch.equal(S, S_eager), f"state differs on replay {r}"


def test_backward_graph_replays_match_eager():
    kda = need_gpu()
    T, H, lengths = 300, 3, [200, 3, 97]
    case(f"graph backward bf16 T={T} H={H} lengths={lengths}")
    sets = []
    for s in (31, 32, 33):
        d = kda_inputs.prefill_inputs(T, H, dtype="bf16", device="cuda", seed=s, lengths=lengths,
                                      h0_std=0.05)
        gen = torch.Generator(device="cuda").manual_seed(s)
        d["do"] = torch.randn(d["v"].shape, generator=gen, device="cuda").to(torch.bfloat16)
        d["dhT"] = torch.randn(d["h0"].shape, generator=gen, device="cuda") * 0.1
        sets.append(d)
    keys = NAMES + ("h0", "do", "dhT")
    st = {n: sets[0][n].clone() for n in keys}
    cu = sets[0]["cu_seqlens"]

    def fn():
        return kda.kda_chunk_bwd(*[st[n] for n in NAMES], st["do"], h0=st["h0"], cu_seqlens=cu,
                                 dhT=st["dhT"])

    g, outs = _capture(fn)
    for r, d in enumerate(sets):
        for n in keys:
            st[n].copy_(d[n])
        g.replay()
        torch.cuda.synchronize()
        ref = kda.kda_chunk_bwd(*[d[n] for n in NAMES], d["do"], h0=d["h0"], cu_seqlens=cu,
                                dhT=d["dhT"])
        torch.cuda.synchronize()
        print(f"  replay {r}", flush=True)
        for name, a, b in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0"), outs, ref):
            assert torch.equal(a, b), f"{name} differs on replay {r}"
