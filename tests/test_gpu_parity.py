"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle,
element by element, on the same seeded inputs.

Tolerance (normwise, max|x - ref| / max|ref| per output tensor): 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs with fp32 state and accumulation.
Small cases span several chunks and a ragged tail; the five workloads run
at full size in the launch configuration the benchmark times: the
16-document workload against the oracle on every (document, head) unit, the
1M-token one on sampled heads.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from gpu_util import TOL, case, check, gpu_prefill, need_gpu, np_, oracle_prefill

pytestmark = pytest.mark.gpu

SMALL = [
    # dtype, lengths, H, h0_std, chunk, split
    ("f32", [128], 2, None, 16, 0),             # the tiny workload, chunk 16
    ("f32", [100], 3, 0.5, 16, 1),
    ("f32", [100], 3, 0.5, 16, 2),
    ("f32", [100], 3, 0.5, 16, 4),
    ("f32", [100], 3, 0.5, 32, 1),
    ("f32", [100], 3, 0.5, 32, 4),
    ("bf16", [100], 3, 0.5, 16, 1),
    ("bf16", [100], 3, 0.5, 32, 1),
    ("bf16", [100], 3, 0.5, 32, 2),
    ("bf16", [100], 3, 0.5, 32, 4),
    ("f32", [0, 1, 37, 16, 100, 5], 2, 0.3, 16, 0),   # varlen with empty docs
    ("f32", [0, 1, 37, 16, 100, 5], 2, 0.3, 32, 0),
    ("bf16", [0, 1, 37, 16, 100, 5], 2, 0.3, 32, 0),
    ("bf16", [1000], 8, None, 0, 0),
    ("bf16", [333, 31, 700], 4, 0.02, 0, 0),
    # 512 tokens or more per sequence on average: the deeper bf16 pipeline
    # (Gram tiles over two iterations), with empty and sub-chunk sequences
    ("bf16", [4000, 0, 1, 15, 16, 17], 2, 0.3, 16, 1),
    ("bf16", [4000, 0, 1, 15, 16, 17], 2, 0.3, 16, 2),
    # the pipelined 32-token kernel (two 16-token sub-tiles): sequences
    # ending in either sub-tile, and shorter than one sub-tile
    ("bf16", [4000, 0, 1, 15, 16, 17], 2, 0.3, 32, 2),
    ("bf16", [33, 47, 48, 63, 64, 65], 3, 0.3, 32, 2),
]


@pytest.mark.parametrize("dtype,lengths,H,h0_std,chunk,split", SMALL)
def test_small_parity(dtype, lengths, H, h0_std, chunk, split):
    kda = need_gpu()
    T = sum(lengths)
    case(f"small dtype={dtype} lengths={lengths} H={H} h0_std={h0_std} chunk={chunk} split={split}")
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=42 + T + H,
                                  lengths=lengths if len(lengths) > 1 else None,
                                  h0_std=h0_std)
    o, hT = gpu_prefill(kda, d, chunk, split)
    ro, rh = oracle_prefill(d)
    check("o", np_(o), ro, TOL[dtype])
    check("h_T", np_(hT), rh, TOL[dtype])


PER_CHUNK = [
    # dtype, chunk, split, T: every kernel variant of the prefill path (the
    # bf16 chunk-16 kernel also with 640 tokens: its deeper schedule)
    ("bf16", 16, 1, 160), ("bf16", 16, 2, 160), ("bf16", 32, 1, 160), ("bf16", 32, 4, 160),
    ("f32", 16, 1, 160), ("f32", 16, 2, 160), ("f32", 32, 4, 160),
    ("bf16", 16, 1, 640), ("bf16", 16, 2, 640),
    ("bf16", 32, 2, 160), ("bf16", 32, 2, 640),
]


@pytest.mark.parametrize("dtype,chunk,split,T", PER_CHUNK)
def test_every_chunk_output_under_slow_decay(dtype, chunk, split, T):
    """Each chunk's output separately, with slow decay (log alpha near 0) so
    that the incoming state carries into every chunk, and a non-zero h0:
    a wrong output in any one chunk (for instance in one unrolled copy of a
    pipelined loop) fails here even when the whole-tensor norm would hide it."""
    kda = need_gpu()
    H = 2
    case(f"per-chunk dtype={dtype} T={T} H={H} chunk={chunk} split={split} decay_mu=-6")
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=4242, h0_std=0.1,
                                  decay_mu=-6.0)
    o, hT = gpu_prefill(kda, d, chunk, split)
    ro, rh = oracle_prefill(d)
    got = np_(o)
    for c in range(T // 16):
        check(f"o[chunk {c}]", got[16 * c:16 * c + 16], ro[16 * c:16 * c + 16], TOL[dtype])
    check("h_T", np_(hT), rh, TOL[dtype])


def test_all_empty_sequences_return_h0():
    kda = need_gpu()
    case("T_total = 0 with three empty documents")
    H = 2
    h0 = torch.randn(3, H, 128, 128, device="cuda")
    z = torch.empty(0, H, 128, dtype=torch.bfloat16, device="cuda")
    b = torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    o, hT = kda.kda_chunk_fwd(z, z, z, z, b, h0=h0, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert o.shape == (0, H, 128)
    assert torch.equal(hT, h0)


def test_workload_tiny_prefill():
    """The tiny workload: T=128, H=2, fp32, chunk 16, h0 = 0."""
    kda = need_gpu()
    case("workload tiny_prefill_T128_H2_f32 chunk=16")
    d = kda_inputs.config_inputs(0, device="cuda")
    o, hT = gpu_prefill(kda, d, chunk=16)
    ro, rh = oracle_prefill(d)
    check("o", np_(o), ro, TOL["f32"])
    check("h_T", np_(hT), rh, TOL["f32"])


def test_workload_prefill_4k():
    """Single-sequence K3-shape prefill, T=4096, H=96, bf16: every head, in
    the default launch and with 32-token chunks."""
    kda = need_gpu()
    d = kda_inputs.config_inputs(1, device="cuda")
    ro, rh = oracle_prefill(d)
    for chunk in (0, 32):
        case(f"workload prefill_T4096_H96_bf16 chunk={chunk or 'default'}")
        o, hT = gpu_prefill(kda, d, chunk)
        check("o", np_(o), ro, TOL["bf16"])
        check("h_T", np_(hT), rh, TOL["bf16"])


def test_workload_decode_batch256():
    """Batched decode: 256 x 96 states, one token, S updated in place."""
    kda = need_gpu()
    case("workload decode_B256_H96_bf16")
    d = kda_inputs.config_inputs(2, device="cuda")
    S0 = np_(d["S"]).copy()
    ro, rS = oracle.decode(np_(d["q"]), np_(d["k"]), np_(d["v"]), np_(d["log_alpha"]),
                           np_(d["beta"]), S0)
    o = kda.kda_decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S"])
    torch.cuda.synchronize()
    check("o", np_(o), ro, TOL["bf16"])
    # the state is fp32 end to end: hold it to the fp32 bar
    check("S", np_(d["S"]), rS, TOL["f32"])


def _per_unit_errors(got, ref, lo, hi):
    """Normwise error of every head over the tokens [lo, hi): max over the
    head's elements of |got - ref| / max over them of |ref| (inputs
    [T, H, D]); returns the H errors."""
    g = np.asarray(got[lo:hi], dtype=np.float64)
    r = np.asarray(ref[lo:hi], dtype=np.float64)
    num = np.abs(g - r).max(axis=(0, 2))
    den = np.abs(r).max(axis=(0, 2))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def test_workload_varlen_16docs():
    """Varlen packed prefill: 16 documents U{512..8192}, per-document h0,
    H=96, bf16.  The fp64 oracle runs the whole workload (every document and
    head), and the error is taken per (document, head) unit -- o over the
    unit's tokens, h_T over its state -- so that a wrong short document or a
    wrong head cannot hide behind a longer one's larger values."""
    kda = need_gpu()
    d = kda_inputs.config_inputs(3, device="cuda")
    cu = d["cu_seqlens"].cpu().numpy().astype(np.int64)
    H = d["q"].shape[1]
    case(f"workload varlen_prefill_16docs_H96_bf16 T={int(cu[-1])}: GPU run")
    o, hT = gpu_prefill(kda, d)
    case("fp64 oracle over all 16 documents x 96 heads")
    ro, rh = oracle_prefill(d)
    go, gh = np_(o), np_(hT)
    assert np.isfinite(go).all() and np.isfinite(gh).all()
    worst = (0.0, None)
    for n in range(len(cu) - 1):
        eo = _per_unit_errors(go, ro, int(cu[n]), int(cu[n + 1]))
        eh = _per_unit_errors(gh.reshape(len(cu) - 1, H, -1), rh.reshape(len(cu) - 1, H, -1),
                              n, n + 1)
        e = np.maximum(eo, eh)
        h = int(np.argmax(e))
        print(f"  doc {n:2d} len {int(cu[n + 1] - cu[n]):5d}: worst head {h} "
              f"o err {eo[h]:.3e}, h_T err {eh[h]:.3e}", flush=True)
        if e[h] > worst[0]:
            worst = (float(e[h]), (n, h))
        bad = np.nonzero(e > TOL["bf16"])[0]
        assert bad.size == 0, f"doc {n}: heads {bad.tolist()} above {TOL['bf16']:.0e}"
    print(f"  worst unit {worst[1]}: {worst[0]:.3e}", flush=True)
    check("o (whole tensor)", go, ro, TOL["bf16"])
    check("h_T (whole tensor)", gh, rh, TOL["bf16"])


def test_workload_prefill_1m_sampled_heads():
    """Long-context prefill, T=1,048,576, H=96, bf16.  Full GPU run; the
    oracle replays all tokens of heads {0, 95} and two seeded heads."""
    kda = need_gpu()
    case("workload prefill_T1048576_H96_bf16: generating inputs on the device")
    d = kda_inputs.config_inputs(4, device="cuda")
    case("workload prefill_T1048576_H96_bf16: GPU run")
    o, hT = gpu_prefill(kda, d)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1004, 98])))
    heads = [0, 95] + [int(x) for x in rng.choice(np.arange(1, 95), size=2, replace=False)]
    sl = lambda t: np_(t[:, heads].contiguous())
    case(f"oracle on heads {heads} over all tokens")
    ro, rh = oracle.fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["log_alpha"]),
                        np_(d["beta"][:, heads].contiguous()), dv_block=32)
    go, gh = np_(o[:, heads].contiguous()), np_(hT[:, heads].contiguous())
    for i, h in enumerate(heads):
        print(f"  head {h}", flush=True)
        check("o", go[:, i], ro[:, i], TOL["bf16"])
        check("h_T", gh[:, i], rh[:, i], TOL["bf16"])
