"""The allocation-free backward entry point (kda_chunk_bwd_noalloc) against
the workspace one (kda_chunk_bwd), through the C ABI: the same kernels on
the same inputs, so every gradient must agree bit for bit; both are also
held to the fp64 reverse-mode oracle's tolerance.  Two calls in a row, the
second on a smaller problem, so the second runs over the scratch the first
left behind; then the first problem again."""
import numpy as np
import pytest
import torch

import kda_inputs
from gpu_util import TOL, case, check, need_gpu, np_

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0")


def _problem(dtype, T, H, lengths, seed):
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=seed, lengths=lengths,
                                  h0_std=0.1)
    g = torch.Generator(device="cuda").manual_seed(seed)
    do = torch.randn((T, H, 128), generator=g, device="cuda").to(d["q"].dtype)
    dhT = torch.randn((d["N"], H, 128, 128), generator=g, device="cuda") * 0.1
    return d, do, dhT


def _compare(kda, dtype, T, H, lengths, seed, with_oracle):
    from oracle import backward as obwd
    case(f"no-alloc backward {dtype} T={T} H={H} lengths={lengths}")
    d, do, dhT = _problem(dtype, T, H, lengths, seed)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], do)
    kw = dict(h0=d["h0"], cu_seqlens=d["cu_seqlens"], dhT=dhT)
    ref = kda.kda_chunk_bwd(*args, **kw)
    got = kda.kda_chunk_bwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, got, ref):
        assert torch.equal(a, b), f"{name}: the no-alloc entry point differs from kda_chunk_bwd"
    if with_oracle:
        cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].cpu().numpy().astype(np.int64)
        oref = obwd.bwd(np_(d["q"]), np_(d["k"]), np_(d["v"]), np_(d["log_alpha"]),
                        np_(d["beta"]), np_(do), dhT=np_(dhT), h0=np_(d["h0"]), cu_seqlens=cu)
        for name, a, r in zip(NAMES, got, oref):
            check(name, np_(a), r, TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_backward_matches_workspace_entry_point(dtype):
    kda = need_gpu()
    _compare(kda, dtype, 300, 4, [100, 0, 200], 71, True)    # first call
    _compare(kda, dtype, 40, 2, [17, 23], 72, True)          # a smaller one after it
    _compare(kda, dtype, 300, 4, [100, 0, 200], 71, False)   # and the first again


def test_noalloc_backward_at_the_size_limit():
    """The largest bf16 shape of the 4096-token, 96-head family inside the
    scratch: 512 tokens x 96 heads ((32 + 2) x 96 table entries)."""
    kda = need_gpu()
    _compare(kda, "bf16", 512, 96, None, 73, False)


def test_noalloc_backward_refuses_oversize_without_launching():
    kda = need_gpu()
    case("no-alloc backward above the scratch limit: refused")
    d, do, dhT = _problem("bf16", 4096, 96, None, 74)
    with pytest.raises(kda.KDAError) as e:
        kda.kda_chunk_bwd_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], do)
    assert e.value.code == 6   # KDA_ERR_WORKSPACE
