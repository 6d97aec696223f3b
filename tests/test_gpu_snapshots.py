"""Prefix snapshots of the state (kda_chunk_fwd_snap) and replay from them,
against the fp64 oracle.

The pages store sparse KDA snapshots at fixed token boundaries for a prefix
cache, restore a snapshot into private state to resume prefill, and, for
speculative decoding, replay only the accepted draft tokens from the
pre-draft state ("From GPT-2 to Kimi K3, from first principles": "Serving a
hybrid cache"; "Speculative decoding cannot naively roll KDA back").  A
snapshot after p tokens of a sequence must equal the oracle's final state of
that sequence's first p tokens, and resuming from it must give the same
outputs as the uninterrupted run.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from gpu_util import TOL, case, check, need_gpu, nerr, np_

pytestmark = pytest.mark.gpu


def _oracle_prefix_state(d, bos, p, n):
    """fp64 oracle state of sequence n (starting at token bos) after p tokens."""
    sl = slice(bos, bos + p)
    h0 = None if d["h0"] is None else np_(d["h0"])[n:n + 1]
    _, hT = oracle.fwd(np_(d["q"][sl]), np_(d["k"][sl]), np_(d["v"][sl]),
                       np_(d["log_alpha"][sl]), np_(d["beta"][sl]), h0=h0)
    return hT[0]


SNAP_CASES = [
    # dtype, lengths, H, interval
    ("bf16", [100, 1000, 37, 512, 1536], 2, 256),
    ("bf16", [100, 1000, 37, 512, 1536], 2, 512),
    ("bf16", [40, 33], 1, 16),                    # every chunk
    ("f32", [100, 1000, 37, 512, 1536], 2, 256),
    ("f32", [300], 2, 32),
    ("bf16", [520] * 8, 32, 256),                 # 256 chains: the whole-head kernel
]


@pytest.mark.parametrize("dtype,lengths,H,interval", SNAP_CASES)
def test_snapshots_match_oracle_prefix_states(dtype, lengths, H, interval):
    kda = need_gpu()
    T = sum(lengths)
    case(f"snapshots dtype={dtype} lengths={lengths} H={H} interval={interval}")
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=77 + T, h0_std=0.1,
                                  lengths=lengths if len(lengths) > 1 else None, decay_mu=-6.0)
    o, hT, snap, snap_cu = kda.kda_chunk_fwd_snap(
        d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], h0=d["h0"],
        cu_seqlens=d["cu_seqlens"], interval=interval)
    torch.cuda.synchronize()
    cu = np.concatenate([[0], np.cumsum(lengths)])
    base = np.zeros(len(lengths) + 1, dtype=np.int64) if snap_cu is None else \
        snap_cu.cpu().numpy().astype(np.int64)
    expect = sum(L // interval for L in lengths)
    assert snap.shape[0] == expect
    got = np_(snap)
    heads = range(H) if H <= 2 else (0, H - 1)
    for n, L in enumerate(lengths):
        for j in range(1, L // interval + 1):
            ref = _oracle_prefix_state(d, int(cu[n]), j * interval, n)
            idx = int(base[n]) + j - 1
            for hh in heads:
                check(f"snap seq {n} after {j * interval} tokens head {hh}", got[idx, hh],
                      ref[hh], TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_replay_from_snapshot_continues_the_run(dtype):
    """Restore a snapshot (read-only) as h0 and resume: outputs and final
    state equal the uninterrupted run's, and the oracle's."""
    kda = need_gpu()
    T, H, interval, p = 1536, 2, 512, 1024
    case(f"replay dtype={dtype} T={T} from snapshot at {p}")
    d = kda_inputs.prefill_inputs(T, H, dtype=dtype, device="cuda", seed=901, decay_mu=-6.0)
    o, hT, snap, _ = kda.kda_chunk_fwd_snap(d["q"], d["k"], d["v"], d["log_alpha"],
                                            d["beta"], interval=interval)
    j = p // interval
    h0 = snap[j - 1:j].clone()
    before = snap.clone()
    sl = slice(p, T)
    o2, hT2 = kda.kda_chunk_fwd(d["q"][sl].contiguous(), d["k"][sl].contiguous(),
                                d["v"][sl].contiguous(), d["log_alpha"][sl].contiguous(),
                                d["beta"][sl].contiguous(), h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(snap, before)          # the snapshot itself is untouched
    check("replayed o vs uninterrupted o", np_(o2), np_(o[sl]), TOL[dtype])
    check("replayed h_T vs uninterrupted h_T", np_(hT2), np_(hT), TOL[dtype])
    ro, rh = oracle.fwd(np_(d["q"]), np_(d["k"]), np_(d["v"]), np_(d["log_alpha"]),
                        np_(d["beta"]))
    check("replayed o vs oracle", np_(o2), ro[sl], TOL[dtype])
    check("replayed h_T vs oracle", np_(hT2), rh, TOL[dtype])


def test_speculative_draft_replays_only_accepted_tokens():
    """A 7-token draft is verified from the state at a snapshot; only the
    first 4 are accepted, and replaying those 4 from the same (unchanged)
    snapshot gives the state after exactly 4 tokens, not 7."""
    kda = need_gpu()
    H, p, draft, accepted = 2, 512, 7, 4
    T = p + draft
    case(f"speculative draft of {draft}, {accepted} accepted, from snapshot at {p}")
    d = kda_inputs.prefill_inputs(T, H, dtype="bf16", device="cuda", seed=902, decay_mu=-6.0)
    _, _, snap, _ = kda.kda_chunk_fwd_snap(d["q"][:p].contiguous(), d["k"][:p].contiguous(),
                                           d["v"][:p].contiguous(),
                                           d["log_alpha"][:p].contiguous(),
                                           d["beta"][:p].contiguous(), interval=p)
    pre = snap[0:1]

    def part(a, b):
        return [d[x][a:b].contiguous() for x in ("q", "k", "v", "log_alpha", "beta")]

    o_verify, _ = kda.kda_chunk_fwd(*part(p, T), h0=pre, store_state=False)
    o_acc, h_acc = kda.kda_chunk_fwd(*part(p, p + accepted), h0=pre)
    torch.cuda.synchronize()
    check("verify pass o (accepted part) vs replay o", np_(o_verify[:accepted]), np_(o_acc),
          TOL["bf16"])
    ro, rh = oracle.fwd(*[np_(d[x][:p + accepted]) for x in ("q", "k", "v", "log_alpha", "beta")])
    check("replayed state after the accepted prefix", np_(h_acc), rh, TOL["bf16"])
    # the state after all 7 draft tokens is a different answer, well outside
    # the tolerance: keeping it would be the error the replay avoids
    _, rh7 = oracle.fwd(*[np_(d[x][:T]) for x in ("q", "k", "v", "log_alpha", "beta")])
    assert nerr(np_(h_acc), rh7) > 5 * TOL["bf16"]


def test_snapshot_entries_past_n_snap_are_not_written():
    """n_snap bounds the writes whatever snap_cu claims: a buffer with two
    guard entries after n_snap keeps them intact."""
    kda = need_gpu()
    lengths, H, interval = [512, 1024], 2, 256
    T = sum(lengths)
    case("snapshot bound: n_snap one short of the count")
    d = kda_inputs.prefill_inputs(T, H, dtype="bf16", device="cuda", seed=903,
                                  lengths=lengths)
    snap_cu, n = kda.snapshot_index(d["cu_seqlens"], T, interval)
    assert n == 6
    buf = torch.full((n + 1, H, 128, 128), 12345.0, dtype=torch.float32, device="cuda")
    kda.kda_chunk_fwd_snap(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                           cu_seqlens=d["cu_seqlens"], interval=interval, snap=buf,
                           snap_cu=snap_cu, n_snap=n - 1)
    torch.cuda.synchronize()
    assert torch.all(buf[n - 1:] == 12345.0)
    assert not torch.any(buf[:n - 1] == 12345.0)
