"""Segment summaries and their scan (kda_segment_summary, kda_segment_scan),
the building blocks of KDA context parallelism, against the fp64 oracle.

Because the KDA state update is affine in the state, a segment of a sequence
maps its incoming state as S_out = M S_in + B, with M the product of the
segment's transitions (I - beta k k^T) Diag(alpha) and B the state reached
from a zero start ("An infra-oriented diagram of Kimi K3": "KDA Context
Parallelism").  Each segment is summarised on its own, an exclusive scan
over the summaries gives the state entering every segment, and a second
prefill pass per segment from that state gives the outputs of the whole
sequence.

Pins: M must equal the oracle's final state of the segment run from h0 = I
with v = 0 (the product of the transitions applied to the identity), B the
oracle's final state from h0 = 0; the scan must match the fp64 recurrence on
seeded random summaries; the reconstructed outputs and boundary states must
match the oracle's uninterrupted run of the whole sequence.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from gpu_util import TOL, case, check, need_gpu, np_

pytestmark = pytest.mark.gpu

D = 128


def _cu(lengths, device="cuda"):
    return torch.as_tensor(kda_inputs.cu_from_lengths(lengths), dtype=torch.int32,
                           device=device)


def _oracle_states(d, lengths, h0=None, v_zero=False, identity=False):
    """fp64 oracle final state of each segment run on its own."""
    cu = kda_inputs.cu_from_lengths(lengths)
    H = d["q"].shape[1]
    out = []
    for n in range(len(lengths)):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        v = np_(d["v"][sl])
        if v_zero:
            v = np.zeros_like(v)
        s0 = np.broadcast_to(np.eye(D), (1, H, D, D)).copy() if identity else h0
        _, hT = oracle.fwd(np_(d["q"][sl]), np_(d["k"][sl]), v, np_(d["log_alpha"][sl]),
                           np_(d["beta"][sl]), h0=s0)
        out.append(hT[0])
    return np.stack(out)


SUMMARY_CASES = [
    # dtype, segment lengths, H   (chains = segments x heads pick the kernel)
    ("bf16", [300, 100, 37, 16, 200], 2),     # ragged tails, few chains
    ("f32", [300, 100, 37, 16, 200], 2),
    ("bf16", [64, 0, 129], 1),                # an empty segment: M = I, B = 0
    ("bf16", [144] * 8, 32),                  # 256 chains: the whole-head kernel
    ("f32", [80] * 4, 64),                    # 256 chains, fp32 inputs
]


@pytest.mark.parametrize("dtype,lengths,H", SUMMARY_CASES)
def test_summary_matches_oracle_transition_and_offset(dtype, lengths, H):
    kda = need_gpu()
    T = sum(lengths)
    case(f"segment summary dtype={dtype} lengths={lengths} H={H}")
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=311 + T,
                                  decay_mu=-6.0)
    M, B = kda.kda_segment_summary(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                   cu_seqlens=_cu(lengths))
    torch.cuda.synchronize()
    assert M.shape == (len(lengths), H, D, D) and B.shape == M.shape
    M_ref = _oracle_states(d, lengths, v_zero=True, identity=True)
    B_ref = _oracle_states(d, lengths)
    heads = range(H) if H <= 2 else (0, H // 2, H - 1)
    gM, gB = np_(M), np_(B)
    for n, L in enumerate(lengths):
        for hh in heads:
            check(f"M seg {n} (len {L}) head {hh}", gM[n, hh], M_ref[n, hh], TOL[dtype])
            if L == 0:
                assert np.array_equal(gM[n, hh], np.eye(D)), "empty segment: M must be I"
                assert not gB[n, hh].any(), "empty segment: B must be 0"
            else:
                check(f"B seg {n} (len {L}) head {hh}", gB[n, hh], B_ref[n, hh], TOL[dtype])


@pytest.mark.parametrize("lengths", [[200, 45], [1500, 3, 700]])
def test_summary_parts_alone_equal_the_pair(lengths):
    """Asking for M or B alone gives the same bits as asking for both (bf16:
    one launch for the pair; both pipeline schedules)."""
    kda = need_gpu()
    H = 2
    case(f"segment summary parts lengths={lengths} H={H}")
    d = kda_inputs.prefill_inputs(sum(lengths), H, dtype="bf16", device="cuda", seed=5)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    cu = _cu(lengths)
    M, B = kda.kda_segment_summary(*args, cu_seqlens=cu)
    M1, none1 = kda.kda_segment_summary(*args, cu_seqlens=cu, want_B=False)
    none2, B1 = kda.kda_segment_summary(*args, cu_seqlens=cu, want_M=False)
    torch.cuda.synchronize()
    assert none1 is None and none2 is None
    assert torch.equal(M, M1) and torch.equal(B, B1)


def _scan_ref(M, B, h0):
    R, H = M.shape[:2]
    S = np.zeros((H, D, D)) if h0 is None else h0.astype(np.float64)
    S_in = np.empty((R, H, D, D))
    for r in range(R):
        S_in[r] = S
        S = np.einsum("hij,hjc->hic", M[r], S) + B[r]
    return S_in, S


@pytest.mark.parametrize("R,H,with_h0", [(1, 1, True), (5, 3, True), (37, 2, False),
                                         (0, 2, True), (8, 96, True)])
def test_scan_matches_fp64_recurrence(R, H, with_h0):
    kda = need_gpu()
    case(f"segment scan R={R} H={H} h0={with_h0}")
    g = np.random.default_rng(1000 + 7 * R + H)
    # contractive transitions (spectral radius below one, like a decayed
    # product of delta-rule factors) and O(1) offsets
    M = (0.9 * np.eye(D) + g.standard_normal((R, H, D, D)) * (0.05 / np.sqrt(D)))
    B = g.standard_normal((R, H, D, D)) * 0.3
    h0 = g.standard_normal((H, D, D)) * 0.5 if with_h0 else None
    M32, B32 = M.astype(np.float32), B.astype(np.float32)
    h032 = None if h0 is None else h0.astype(np.float32)
    S_in, S_fin = kda.kda_segment_scan(
        torch.from_numpy(M32).cuda(), torch.from_numpy(B32).cuda(),
        None if h032 is None else torch.from_numpy(h032).cuda())
    torch.cuda.synchronize()
    ref_in, ref_fin = _scan_ref(M32.astype(np.float64), B32.astype(np.float64),
                                None if h032 is None else h032.astype(np.float64))
    assert S_in.shape == (R, H, D, D) and S_fin.shape == (H, D, D)
    if R:
        check("S_in", np_(S_in), ref_in, 1e-5)
    check("S_final", np_(S_fin), ref_fin, 1e-5)
    if R:
        # the first entry is h0 (or zero) exactly
        first = np_(S_in)[0]
        assert np.array_equal(first, h032 if h032 is not None else np.zeros_like(first))


CP_CASES = [
    # dtype, T, H, segment lengths
    ("bf16", 1000, 2, [300, 100, 400, 200]),
    ("f32", 1000, 2, [300, 100, 400, 200]),
    ("bf16", 777, 2, [17, 256, 1, 503]),      # ragged: a one-token segment
    ("bf16", 2048, 64, [512, 512, 512, 512]),  # 256 chains in the summary
]


@pytest.mark.parametrize("dtype,T,H,lengths", CP_CASES)
def test_context_parallel_reconstruction(dtype, T, H, lengths):
    """Summaries -> scan -> second pass per segment equals the oracle's
    uninterrupted run of the whole sequence (outputs, boundary states and
    final state)."""
    kda = need_gpu()
    assert sum(lengths) == T
    case(f"context parallel dtype={dtype} T={T} H={H} segments={lengths}")
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=4242 + T,
                                  h0_std=0.1, decay_mu=-6.0)
    cu = _cu(lengths)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    M, B = kda.kda_segment_summary(*args, cu_seqlens=cu)
    S_in, S_final = kda.kda_segment_scan(M, B, d["h0"])
    o2, hT2 = kda.kda_chunk_fwd(*args, h0=S_in, cu_seqlens=cu)
    torch.cuda.synchronize()

    heads = list(range(H)) if H <= 2 else [0, H - 1]
    hsel = torch.as_tensor(heads)
    sub = {x: d[x][:, hsel].contiguous() for x in ("q", "k", "v", "log_alpha", "beta")}
    h0s = np_(d["h0"])[:, heads]
    o_ref, hT_ref = oracle.fwd(*(np_(sub[x]) for x in ("q", "k", "v", "log_alpha", "beta")),
                               h0=h0s)
    check("o (reconstructed)", np_(o2)[:, heads], o_ref, TOL[dtype])
    check("S_final", np_(S_final)[heads], hT_ref[0], TOL[dtype])
    check("h_T of the last segment", np_(hT2)[-1, heads], hT_ref[0], TOL[dtype])
    cu_np = kda_inputs.cu_from_lengths(lengths)
    for r in range(1, len(lengths)):
        p = int(cu_np[r])
        _, ref = oracle.fwd(*(np_(sub[x][:p]) for x in ("q", "k", "v", "log_alpha", "beta")),
                            h0=h0s)
        check(f"S_in[{r}] (after {p} tokens)", np_(S_in)[r, heads], ref[0], TOL[dtype])


def test_context_parallel_full_size_sampled():
    """One GPU's share of a 1M-token sequence split over 8 ranks (131072
    tokens, 96 heads, bf16), cut into 8 segments of 16384: the scan-stitched
    final state and the outputs of sampled tokens agree with the plain
    single-pass prefill of the same share (the oracle pins the two paths at
    the smaller sizes above), and the sampled heads' final state with the
    oracle."""
    kda = need_gpu()
    T, H, R = 131072, 96, 8
    lengths = [T // R] * R
    case(f"context parallel full size T={T} H={H} R={R}")
    d = kda_inputs.prefill_inputs(T, H, dtype="bf16", device="cuda", seed=8080)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    cu = _cu(lengths)
    M, B = kda.kda_segment_summary(*args, cu_seqlens=cu)
    S_in, S_final = kda.kda_segment_scan(M, B, None)
    o2, _ = kda.kda_chunk_fwd(*args, h0=S_in, cu_seqlens=cu)
    o1, hT1 = kda.kda_chunk_fwd(*args)
    torch.cuda.synchronize()
    check("S_final vs single pass", np_(S_final), np_(hT1)[0], TOL["bf16"])
    rows = torch.as_tensor(np.random.default_rng(3).choice(T, 512, replace=False))
    check("sampled o vs single pass", np_(o2[rows]), np_(o1[rows]), TOL["bf16"])
    heads = [0, 95]
    hsel = torch.as_tensor(heads)
    sub = [np_(d[x][:, hsel].contiguous()) for x in ("q", "k", "v", "log_alpha", "beta")]
    _, hT_ref = oracle.fwd(*sub)
    check("S_final sampled heads vs oracle", np_(S_final)[heads], hT_ref[0], TOL["bf16"])
