#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one chunkwise prefill (kda_chunk_fwd) of the K3-shape
single-sequence workload: T = 4096 tokens, H = 96 heads, d_k = d_v = 128,
bf16 inputs, fp32 state, h0 = 0 (the workload the headline "KDA prefill
tokens/s @H=96, d=128" is quoted on).  Inputs are seeded synthetic tensors
resident in HBM before timing; two input sets alternate so that consecutive
steps do not hit in the 256 MiB Infinity Cache.  The decode half of the
metric (decode state GB/s) is measured in the same run on the batched
decode workload (256 sequences x 96 heads, one token each, state updated in
place) and reported under "decode".  The other three workloads -- the tiny
fp32 prefill, the 16-document varlen prefill and the 1M-token sequence (a
few steps) -- are timed too, under "other_workloads", each with the CPU
oracle's rate beside it, and a 1 GiB device copy gives the measured
streaming ceiling beside the 8 TB/s peak.

Prints ONE JSON line.  `--gpus N` with N > 1 exits: this build is single-GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s @H=96,d=128 (% MFMA peak); decode state GB/s (% HBM)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (2.5 PFLOP/s)
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (vector / MFMA)
MFMA_TARGET = 0.40             # the prefill target: >= 40% of bf16 MFMA peak
RUN_CHUNK = 16                 # tokens per chunk of the default bf16 prefill kernel
D = 128


def flops_per_head_token(C=64):
    """Algorithmic flops per (token, head) of chunkwise KDA counted at chunk
    length C: 6 d^2 for the three state products plus the causal halves of
    the chunk-local products and the triangular solve."""
    return 6 * D * D + D * (5 * C + 3) + C * C / 3.0


def decode_bytes(B, H, esize=2):
    """Algorithmic HBM bytes of one decode step: every (sequence, head) state
    read and written once (128 x 128 fp32 each way) plus the token's q, k,
    v, log_alpha, beta in and o out."""
    return B * H * (D * D * 4 * 2 + esize * (4 * D + 1 + D))


def prefill_bytes(T, H, N, esize=2, h0=False):
    """Algorithmic HBM bytes of one prefill: q, k, v, log_alpha (d each),
    beta, o (d) per (token, head), plus 64 KiB per (sequence, head) for h_T
    (and h0 when given)."""
    per_ht = esize * (4 * D + 1 + D)
    state = N * H * D * D * 4
    return T * H * per_ht + state * (2 if h0 else 1)


def kernel_source_hash():
    # the kernel sources and the build script (which holds the compiler flags)
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "gated_delta_rule_27_amd")
    csrc = os.path.join(pkg, "csrc")
    paths = [os.path.join(csrc, fn) for fn in sorted(os.listdir(csrc))]
    for p in paths + [os.path.join(pkg, "build.py")]:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(name, src_hash):
    """HBM bytes per launch measured with rocprofv3 counters, from the
    committed summary; None if absent or taken on another kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_launches(fn, steps, warmup, stream, ahead=False):
    """Run fn `warmup` times, then `steps` times with a HIP event pair around
    each launch on `stream`; returns (wall seconds, per-launch ms list).

    With `ahead`, for kernels shorter than the host's own cost of a launch
    through Python: each group of launches is queued behind a spin kernel
    long enough for the host to enqueue the whole group, and a launch's time
    is the spacing of its end event from the previous launch's end event in
    the same group (the first launch of a group only opens it), so that the
    host's gaps are not counted (wall is then None).  Callers of the ahead
    mode take the median of the spacings: now and then (MI355X, ROCm 7.2)
    a queue stalls for tens of milliseconds between two launches, one long
    gap among back-to-back kernels, which alone would dominate the mean of
    a 50 us kernel."""
    import torch
    th = time.perf_counter()
    for i in range(warmup):
        fn(i)
    host_ms = (time.perf_counter() - th) * 1e3 / max(warmup, 1)
    torch.cuda.synchronize()
    if ahead:
        cyc_per_ms = sleep_rate(torch, stream)
        group = 21
        out = []
        done = 0
        while done < steps:
            n = min(group, steps - done + 1)
            ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
            torch.cuda._sleep(int(cyc_per_ms * (3.0 * n * host_ms + 0.5)))
            for j in range(n):
                fn(warmup + done + j)
                ends[j].record(stream)
            torch.cuda.synchronize()
            out += [ends[j - 1].elapsed_time(ends[j]) for j in range(1, n)]
            done += n - 1
        return None, out
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        fn(warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in ev]


_SLEEP_RATE = []


def sleep_rate(torch, stream):
    """Counter cycles per millisecond of torch's spin kernel on this GPU."""
    if not _SLEEP_RATE:
        cyc = 20_000_000
        torch.cuda._sleep(cyc // 10)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.cuda._sleep(cyc)
        e1.record(stream)
        torch.cuda.synchronize()
        _SLEEP_RATE.append(cyc / max(e0.elapsed_time(e1), 1e-3))
    return _SLEEP_RATE[0]


def host_info():
    """CPU model and host memory, for the record."""
    model, mem_gib = None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    mem_gib = round(int(line.split()[1]) / 2**20, 1)
                    break
    except OSError:
        pass
    return model, mem_gib


def cpu_baseline(T, H):
    """The CPU oracle on the whole prefill workload, on this host: fp32, the
    median of three runs (the reported value), and one fp64 run."""
    import kda_inputs
    import oracle
    d = kda_inputs.prefill_inputs(T, H, dtype="bf16", device="cpu", seed=1001)
    args = [kda_inputs.to_numpy(d[k]) for k in ("q", "k", "v", "log_alpha", "beta")]
    threads = oracle.default_threads()
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.fwd(*args, precision="f32", nthreads=threads)
        runs.append(time.perf_counter() - t0)
    dt = sorted(runs)[1]
    t0 = time.perf_counter()
    oracle.fwd(*args, precision="f64", nthreads=threads)
    dt64 = time.perf_counter() - t0
    model, mem_gib = host_info()
    return {"value": round(T / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole prefill workload (T={T}, H={H}, d=128), fp32 oracle, median of "
                      f"3 runs {dt:.2f} s wall",
            "fp64_tokens_per_s": round(T / dt64, 1), "cpu_model": model, "host_mem_gib": mem_gib}


def cpu_oracle_rows(kind):
    """The CPU oracle of another row of the path, timed on a bounded sample of
    its workload on this host (a reported baseline, never tuned): returns
    {value, unit, cores, kind, sample}.  Single-threaded NumPy for the layer
    and the backward (their oracles are plain NumPy), the multithreaded C
    oracle for decode."""
    import kda_inputs
    import oracle
    n = kda_inputs.to_numpy
    if kind == "decode":
        B, H = 64, 96
        d = kda_inputs.decode_inputs(B, H, dtype="bf16", device="cpu", seed=2001)
        args = [n(d[x]) for x in ("q", "k", "v", "log_alpha", "beta", "S")]
        t0 = time.perf_counter()
        oracle.decode(*args, precision="f32")
        dt = time.perf_counter() - t0
        state = B * H * 128 * 128 * 4 * 2
        return {"value": round(state / dt / 1e9, 2), "unit": "state GB/s",
                "cores": oracle.default_threads(), "kind": "oracle",
                "sample": f"{B} sequences x {H} heads, fp32 C oracle, {dt:.2f} s"}
    if kind == "backward":
        from oracle import backward as obwd
        T, H = 1024, 2
        d = kda_inputs.prefill_inputs(T, H, dtype="bf16", device="cpu", seed=2002)
        do = n(kda_inputs.prefill_inputs(T, H, dtype="bf16", device="cpu", seed=2003)["v"])
        t0 = time.perf_counter()
        obwd.bwd(*(n(d[x]) for x in ("q", "k", "v", "log_alpha", "beta")), do)
        dt = time.perf_counter() - t0
        return {"value": round(T * H / dt, 1), "unit": "token-heads/s", "cores": 1,
                "kind": "oracle", "sample": f"T={T}, {H} heads, float64 NumPy oracle, {dt:.2f} s"}
    if kind == "layer":
        from oracle import layer as olayer
        T, H = 512, 96
        d = kda_inputs.layer_inputs(T, H, dtype="bf16", device="cpu", seed=2004)
        t0 = time.perf_counter()
        olayer.prologue(*(n(d[x]) for x in ("xq", "xk", "xv", "a_raw", "b_raw", "conv_w",
                                            "a_bias")))
        olayer.epilogue(n(d["o"]), n(d["g"]), n(d["norm_w"]))
        dt = time.perf_counter() - t0
        return {"value": round(T / dt, 1), "unit": "tokens/s (prologue + epilogue)", "cores": 1,
                "kind": "oracle", "sample": f"T={T}, {H} heads, float64 NumPy oracle, {dt:.2f} s"}
    raise ValueError(kind)


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def copy_bandwidth(torch, dev, stream):
    """A plain device copy of 1 GiB (read + write), timed with HIP events:
    the practical streaming ceiling of this GPU, beside the 8 TB/s peak."""
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    gbps = 5 * 2 * src.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return round(gbps, 1)


def mfma_fracs(T, H, ms, chunk_run=RUN_CHUNK, peak_tflops=BF16_PEAK_TFLOPS):
    """%MFMA of a prefill taking `ms`: at the chunk length the kernel runs
    (the flops it executes) and, labelled, at F(64) (a fixed yardstick
    that does not move with the chunk length; it counts more chunk-local
    work than a 16-token kernel does)."""
    f_run = T * H * flops_per_head_token(chunk_run)
    f64 = T * H * flops_per_head_token(64)
    s = ms * 1e-3 * peak_tflops * 1e12
    return {"chunk_run": chunk_run, "mfma_frac_at_run_chunk": round(f_run / s, 4),
            "mfma_frac_F64": round(f64 / s, 4)}


def oracle_rate_prefill(d, heads=None, dv_block=0):
    """The fp32 CPU oracle on a prefill workload (all heads, or the listed
    heads of a one-sequence workload), one run, on this host's cores:
    returns (seconds, head-tokens processed, threads)."""
    import kda_inputs
    import oracle
    n = kda_inputs.to_numpy
    names = ("q", "k", "v", "log_alpha", "beta")
    if heads is None:
        args = [n(d[x]) for x in names]
        cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].cpu().numpy()
        h0 = n(d["h0"]) if d["h0"] is not None else None
    else:
        args = [n(d[x][:, heads].contiguous()) for x in names]
        cu, h0 = None, None
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.fwd(*args, h0=h0, cu_seqlens=cu, precision="f32", nthreads=threads,
               dv_block=dv_block, store_state=True)
    dt = time.perf_counter() - t0
    return dt, args[0].shape[0] * args[0].shape[1], threads


def extra_prefill(torch, kda, kda_inputs, dev, stream, cfg_id, steps, warmup, cpu=True):
    """Timing line of another prefill workload (same kernel path, its default
    configuration, or the chunk length the workload fixes): tokens/s, HBM
    fraction, %MFMA, and the CPU oracle beside it (the whole workload, or the
    1M-token workload's four sampled heads with the per-head rate and a
    labelled whole-workload extrapolation)."""
    cfg = kda_inputs.CONFIGS[cfg_id]
    print(f"[bench] {cfg['name']}: generating inputs", file=sys.stderr, flush=True)
    d = kda_inputs.config_inputs(cfg_id, device=dev)
    T, H = d["q"].shape[0], d["q"].shape[1]
    N = 1 if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    o = torch.empty_like(d["v"])
    hT = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    chunk = cfg.get("chunk") or 0
    esize = d["q"].element_size()

    def step(i):
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], h0=d["h0"],
                          cu_seqlens=d["cu_seqlens"], o=o, h_T=hT, chunk=chunk)

    print(f"[bench] {cfg['name']}: timing", file=sys.stderr, flush=True)
    wall, ms = time_launches(step, steps, warmup, stream)
    avg = sum(ms) / len(ms)
    nbytes = prefill_bytes(T, H, N, esize=esize, h0=d["h0"] is not None)
    out = {"workload": cfg["name"], "T": T, "H": H, "sequences": N, "dtype": cfg["dtype"],
           "steps": steps, "warmup": warmup,
           "tokens_per_s": round(T * steps / wall, 1), "kernel_ms": round(avg, 4),
           "kernel_ms_median": round(median(ms), 4),
           "hbm_frac": round(nbytes / (avg * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
           "algorithmic_bytes": nbytes}
    if cfg["dtype"] == "bf16":
        out.update(mfma_fracs(T, H, avg))
    else:   # fp32 operands run on the fp32 MFMA
        out.update(mfma_fracs(T, H, avg, chunk_run=chunk or RUN_CHUNK,
                              peak_tflops=FP32_PEAK_TFLOPS))
        out["mfma_peak"] = "fp32 157.3 TFLOP/s"
    if cpu:
        print(f"[bench] {cfg['name']}: CPU oracle", file=sys.stderr, flush=True)
        if cfg_id == 4:
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1004, 98])))
            heads = [0, 95] + [int(x) for x in rng.choice(np.arange(1, 95), size=2,
                                                           replace=False)]
            secs, ht, thr = oracle_rate_prefill(d, heads=heads, dv_block=32)
            per_head = ht / secs
            out["cpu_oracle"] = {
                "value": round(per_head, 1), "unit": "head-tokens/s", "cores": thr,
                "kind": "oracle",
                "sample": f"heads {heads} x all {T} tokens, fp32 C oracle, one run "
                          f"{secs:.2f} s wall (value-column blocks of 32 as units)",
                "extrapolated_tokens_per_s_all_96_heads": round(per_head / H, 2),
                "extrapolation": "per-head rate / 96 heads, assuming the same rate per head"}
        else:
            runs = 3 if T * H < 100000 else 1
            best = []
            for _ in range(runs):
                secs, ht, thr = oracle_rate_prefill(d)
                best.append(secs)
            secs = sorted(best)[len(best) // 2]
            out["cpu_oracle"] = {
                "value": round(T / secs, 1), "unit": "tokens/s", "cores": thr, "kind": "oracle",
                "sample": f"whole workload (T={T}, H={H}, {N} sequences), fp32 C oracle, "
                          f"{'median of 3 runs' if runs == 3 else 'one run'} {secs:.3f} s wall"}
    del d, o, hT
    torch.cuda.empty_cache()
    return out


def verify_replay(torch, kda, kda_inputs, dev, stream, steps, warmup):
    """Batched speculative decoding: 256 requests x 96 heads, each with its
    cached fp32 state; a 7-token draft is verified (outputs only, state
    untouched), then the 4 accepted tokens are replayed from the same states
    (new states written).  Measured with the multi-token recurrent kernel
    (kda_decode_multi) and, for comparison, with the chunk path; 7
    single-token decode steps would read and write every state 7 times."""
    B, H, draft, acc = 256, 96, 7, 4
    d = kda_inputs.prefill_inputs(B * draft, H, dtype="bf16", device=dev, seed=1005,
                                  lengths=[draft] * B, h0_std=0.02)
    names = ("q", "k", "v", "log_alpha", "beta")
    w = {x: d[x].view(B, draft, *d[x].shape[1:]) for x in names}
    n_acc = torch.full((B,), acc, dtype=torch.int32, device=dev)
    S_new = d["h0"].clone()
    o = torch.empty((B, draft, H, D), dtype=torch.bfloat16, device=dev)

    def mverify(i):
        kda.kda_decode_multi(*[w[x] for x in names], d["h0"], update_state=False, o=o)

    def mreplay(i):
        # each timed replay updates S_new again: the same work every time
        kda.kda_decode_multi(*[w[x] for x in names], S_new, n_acc, update_state=True, o=o)

    # chunk path: accepted tokens packed as sequences of `acc`
    dr = {x: w[x][:, :acc].reshape(B * acc, *d[x].shape[1:]).contiguous() for x in names}
    dr["cu_seqlens"] = torch.arange(0, B * acc + 1, acc, dtype=torch.int32, device=dev)
    oc = torch.empty_like(d["v"])
    oc_r = torch.empty_like(dr["v"])
    h_new = torch.empty_like(d["h0"])

    def cverify(i):
        kda.kda_chunk_fwd(*[d[x] for x in names], h0=d["h0"], cu_seqlens=d["cu_seqlens"],
                          o=oc, store_state=False)

    def creplay(i):
        kda.kda_chunk_fwd(*[dr[x] for x in names], h0=d["h0"], cu_seqlens=dr["cu_seqlens"],
                          o=oc_r, h_T=h_new)

    res = {}
    for name, fn in (("multi_verify", mverify), ("multi_replay", mreplay),
                     ("chunk_verify", cverify), ("chunk_replay", creplay)):
        _, ms = time_launches(fn, steps, warmup, stream, ahead=True)
        res[name] = median(ms)
    state = B * H * D * D * 4
    out = {"requests": B, "H": H, "draft_tokens": draft, "accepted": acc,
           "kernel": "kda::decode_multi_kernel",
           "verify_ms": round(res["multi_verify"], 4), "replay_ms": round(res["multi_replay"], 4),
           "verify_state_read_GBps": round(state / (res["multi_verify"] * 1e-3) / 1e9, 1),
           "replay_state_GBps": round(2 * state / (res["multi_replay"] * 1e-3) / 1e9, 1),
           "chunk_path_verify_ms": round(res["chunk_verify"], 4),
           "chunk_path_replay_ms": round(res["chunk_replay"], 4)}
    del d, w, dr, o, oc, oc_r, h_new, S_new
    torch.cuda.empty_cache()
    return out


def context_parallel(torch, kda, kda_inputs, dev, stream, steps, warmup):
    """One rank's share of KDA context parallelism for a 1M-token sequence
    over 8 ranks: 131072 tokens x 96 heads, bf16.  The rank summarises its
    segment (M and B: in bf16 one launch whose state waves run both passes
    over shared operands; each alone is timed too), the scan over the 8
    summaries gives its incoming state (here the local summary stands in for
    the 7 others, which would arrive by an all-gather), and a second prefill
    pass from that state gives its outputs.  Timed beside one plain prefill
    pass over the same share."""
    T, H, R = 131072, 96, 8
    d = kda_inputs.prefill_inputs(T, H, dtype="bf16", device=dev, seed=1006)
    args = [d[x] for x in ("q", "k", "v", "log_alpha", "beta")]
    o = torch.empty_like(d["v"])
    hT = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    M, B = kda.kda_segment_summary(*args)
    Mr = M.expand(R, H, D, D).contiguous()
    Br = B.expand(R, H, D, D).contiguous()
    S_in, S_fin = kda.kda_segment_scan(Mr, Br)
    h_in = S_in[R - 1:R].contiguous()

    def summary_MB(i):
        kda.kda_segment_summary(*args)

    def summary_B(i):
        kda.kda_segment_summary(*args, want_M=False)

    def summary_M(i):
        kda.kda_segment_summary(*args, want_B=False)

    def scan(i):
        kda.kda_segment_scan(Mr, Br)

    def pass2(i):
        kda.kda_chunk_fwd(*args, h0=h_in, o=o, h_T=hT)

    def plain(i):
        kda.kda_chunk_fwd(*args, o=o, h_T=hT)

    res = {}
    for name, fn in (("summary_MB", summary_MB), ("summary_B", summary_B),
                     ("summary_M", summary_M), ("scan", scan), ("pass2", pass2), ("plain", plain)):
        _, ms = time_launches(fn, steps, warmup, stream, ahead=True)
        res[name] = median(ms)
    tok = T * H * 2
    state = H * D * D * 4
    total = res["summary_MB"] + res["scan"] + res["pass2"]
    out = {"workload": "kda_cp_rank_share_T131072_of_1M_8ranks_H96_bf16", "T": T, "H": H,
           "segments_scanned": R,
           "summary_MB_ms": round(res["summary_MB"], 4),
           "summary_B_ms": round(res["summary_B"], 4), "summary_M_ms": round(res["summary_M"], 4),
           "scan_ms": round(res["scan"], 4), "pass2_ms": round(res["pass2"], 4),
           "plain_prefill_ms": round(res["plain"], 4),
           "rank_total_ms": round(total, 4),
           "rank_tokens_per_s": round(T / (total * 1e-3), 1),
           "vs_plain_prefill": round(total / res["plain"], 3),
           # k, v, log_alpha, beta read; B written | k, log_alpha, beta read; M written
           "summary_B_hbm_frac": round((tok * (3 * D + 1) + state) / (res["summary_B"] * 1e-3)
                                       / (HBM_PEAK_GBS * 1e9), 4),
           "summary_M_hbm_frac": round((tok * (2 * D + 1) + state) / (res["summary_M"] * 1e-3)
                                       / (HBM_PEAK_GBS * 1e9), 4),
           "scan_GBps": round(R * 3 * state / (res["scan"] * 1e-3) / 1e9, 1)}
    del d, args, o, hT, M, B, Mr, Br, S_in, S_fin, h_in
    torch.cuda.empty_cache()
    return out


def layer_elementwise(torch, kda, kda_inputs, dev, stream, steps, warmup, chunk_ms, decode_ms):
    """The prologue (short conv + Swish + L2 norm, decay and write gates) and
    the epilogue (head RMSNorm x output gate) around the core, on the
    4096-token prefill workload and on a 256-request decode step (with the
    convolution history read and written).  HBM fractions count the
    algorithmic bytes: every input read once, every output written once.
    Both kernels are shorter than a launch through the Python binding, so
    they are timed with the GPU kept ahead of the host."""
    out = {}
    for name, T, H, lengths in (("prefill_T4096_H96_bf16", 4096, 96, None),
                                ("decode_B256_H96_bf16", 256, 96, [1] * 256)):
        d = kda_inputs.layer_inputs(T, H, dtype="bf16", device=dev, seed=1007, lengths=lengths,
                                    conv_state=lengths is not None)
        so = torch.empty_like(d["conv_state"]) if d["conv_state"] is not None else None
        y = torch.empty_like(d["o"])

        def pro(i):
            kda.kda_prologue(d["xq"], d["xk"], d["xv"], d["a_raw"], d["b_raw"], d["conv_w"],
                             d["a_bias"], cu_seqlens=d["cu_seqlens"], conv_state=d["conv_state"],
                             store_state=so is not None, state_out=so)

        def epi(i):
            kda.kda_epilogue(d["o"], d["g"], d["norm_w"], y=y)

        _, pms = time_launches(pro, steps, warmup, stream, ahead=True)
        _, ems = time_launches(epi, steps, warmup, stream, ahead=True)
        pavg, eavg = median(pms), median(ems)
        row = H * D * 2
        hist = 0 if so is None else 2 * d["N"] * 9 * row      # history read + written
        pbytes = T * (8 * row + 4 * H) + hist + (3 * 4 + 1) * H * D * 4
        ebytes = T * 3 * row + H * D * 4
        core = chunk_ms if lengths is None else decode_ms
        out[name] = {"prologue_ms": round(pavg, 5), "epilogue_ms": round(eavg, 5),
                     "prologue_hbm_frac": round(pbytes / (pavg * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                     "epilogue_hbm_frac": round(ebytes / (eavg * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                     "prologue_bytes": pbytes, "epilogue_bytes": ebytes,
                     "core_ms": round(core, 5) if core else None,
                     "layer_ms": round(pavg + eavg + core, 5) if core else None}
        del d, so, y
    torch.cuda.empty_cache()
    return out


def backward(torch, kda, kda_inputs, dev, stream, steps, warmup, fwd_ms):
    """Backward pass (kda_chunk_bwd) of the 4096-token, 96-head workload:
    the forward state recursion again (states after every chunk), the
    reverse recursion of the state gradient, and every chunk's gradients.
    Algorithmic bytes: the forward inputs and dout read, the five token
    gradients written (10 rows of 256 B per token and head, plus beta and
    dbeta); the per-chunk state tables are extra traffic of this design."""
    T, H = 4096, 96
    d = kda_inputs.prefill_inputs(T, H, dtype="bf16", device=dev, seed=1008)
    do = torch.randn((T, H, D), device=dev).to(torch.bfloat16)
    ws = torch.empty(kda.kda_chunk_bwd_workspace_size(T, 1, H), dtype=torch.uint8, device=dev)

    def step(i):
        kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], do, workspace=ws)

    wall, ms = time_launches(step, steps, warmup, stream)
    avg = sum(ms) / len(ms)
    alg = T * H * (10 * D * 2 + 4)
    out = {"workload": "kda_backward_T4096_H96_d128_bf16", "ms_per_step": round(avg, 4),
           "tokens_per_s": round(T * steps / wall, 1), "vs_forward": round(avg / fwd_ms, 2),
           "algorithmic_bytes": alg, "state_table_bytes": ws.numel(),
           "hbm_frac_algorithmic": round(alg / (avg * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}
    del d, do, ws
    torch.cuda.empty_cache()
    return out


def decode_section(torch, kda, kda_inputs, dev, stream, steps, warmup, H=96):
    """The batched decode workload: 256 x 96 fp32 states, one bf16 token
    each, the state updated in place (the decode half of the metric)."""
    B = 256
    dd = kda_inputs.decode_inputs(B, H, dtype="bf16", device=dev, seed=1002)
    od = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)

    def dstep(i):
        kda.kda_decode_step(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                            dd["S"], o=od)

    _, dms = time_launches(dstep, steps, warmup, stream)
    davg = sum(dms) / len(dms)
    state_bytes = B * H * D * D * 4 * 2
    total_bytes = decode_bytes(B, H)
    del dd
    torch.cuda.empty_cache()
    return {
        "workload": "kda_decode_B256_H96_d128_bf16", "steps": steps, "warmup": warmup,
        "state_GBps": round(state_bytes / (davg * 1e-3) / 1e9, 1),
        "total_GBps": round(total_bytes / (davg * 1e-3) / 1e9, 1),
        "ms_per_step": round(davg, 5),
        "roofline": {"bound": "hbm",
                     "achieved": round(total_bytes / (davg * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(total_bytes / (davg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("decode_B256_H96_bf16", kernel_source_hash()),
                     "kernel": "kda::decode_kernel",
                     "kernel_ms_median": round(median(dms), 5)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--chunk", type=int, default=0, help="override the chunk length")
    ap.add_argument("--split", type=int, default=0, help="override the column split")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy three times, as the "
                         "reference kernel for scaling HBM byte counters")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip everything but the headline prefill and decode lines")
    ap.add_argument("--skip-long", action="store_true",
                    help="skip the 1M-token single-sequence prefill (129 GB of HBM)")
    ap.add_argument("--long-steps", type=int, default=3,
                    help="timed steps of the 1M-token prefill (one untimed step first)")
    ap.add_argument("--section", default=None,
                    choices=["prefill", "long", "varlen", "tiny", "decode", "backward", "layer",
                             "context_parallel", "verify_replay"],
                    help="time only this section (one JSON object), e.g. under a profiler")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested); "
              "the path is not sharded across GPUs", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_27_amd as kda
    import kda_inputs

    if not torch.cuda.is_available():
        print("bench.py: no ROCm device", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_27_amd import build
        build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    T, H, N = 4096, 96, 1

    def headline_inputs():
        return [kda_inputs.prefill_inputs(T, H, dtype="bf16", device=dev, seed=s)
                for s in (1001, 1101)]

    if args.section:
        if args.section == "prefill":
            sets = headline_inputs()
            o = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)

            def pstep(i):
                d = sets[i % 2]
                kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                  chunk=args.chunk, dv_split=args.split, o=o, store_state=True)

            _, ms = time_launches(pstep, args.steps, args.warmup, stream)
            avg = sum(ms) / len(ms)
            res = {"workload": "kda_prefill_T4096_H96_d128_bf16", "kernel_ms": round(avg, 5),
                   "hbm_frac": round(prefill_bytes(T, H, N) / (avg * 1e-3)
                                     / (HBM_PEAK_GBS * 1e9), 4)}
            res.update(mfma_fracs(T, H, avg))
        elif args.section in ("long", "varlen", "tiny"):
            cid = {"tiny": 0, "varlen": 3, "long": 4}[args.section]
            st = args.long_steps if cid == 4 else args.steps
            res = extra_prefill(torch, kda, kda_inputs, dev, stream, cid, st,
                                1 if cid == 4 else args.warmup, cpu=False)
        elif args.section == "decode":
            res = decode_section(torch, kda, kda_inputs, dev, stream, args.steps, args.warmup)
        elif args.section == "backward":
            res = backward(torch, kda, kda_inputs, dev, stream, args.steps, args.warmup, 1.0)
            res.pop("vs_forward")
        elif args.section == "layer":
            res = layer_elementwise(torch, kda, kda_inputs, dev, stream, args.steps, args.warmup,
                                    None, None)
        elif args.section == "context_parallel":
            res = context_parallel(torch, kda, kda_inputs, dev, stream, args.steps, args.warmup)
        else:
            res = verify_replay(torch, kda, kda_inputs, dev, stream, args.steps, args.warmup)
        print(json.dumps({"section": args.section, "kernel_source_hash": kernel_source_hash(),
                          **res}), flush=True)
        return

    # Decode is timed first: it is half of the metric, and it also brings the
    # GPU to its working clocks before the prefill's own warm-up steps.
    sets = headline_inputs()
    decode_out = None
    if not args.no_decode:
        decode_out = decode_section(torch, kda, kda_inputs, dev, stream, args.steps, args.warmup)

    # ---------------- prefill: T=4096, H=96, bf16 ----------------
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)

    def step(i):
        d = sets[i % 2]
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                          chunk=args.chunk, dv_split=args.split, o=o, h_T=hT)

    wall, ms = time_launches(step, args.steps, args.warmup, stream)
    assert torch.isfinite(o.float()).all().item(), "non-finite prefill output"
    avg_ms = sum(ms) / len(ms)
    tokens_per_s = T * args.steps / wall
    nbytes = prefill_bytes(T, H, N)
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = read_traffic("chunk_fwd_T4096_H96_bf16", src_hash)
    fr = mfma_fracs(T, H, avg_ms, chunk_run=args.chunk or RUN_CHUNK)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_prefill_T4096_H96_d128_bf16", "T": T, "H": H, "d": D,
                   "sequences": N, "h0": "zero", "chunk": args.chunk or "auto",
                   "dv_split": args.split or "auto"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "kda::chunk_ws2_kernel",
                     "kernel_ms": round(avg_ms, 5), "kernel_ms_median": round(median(ms), 5),
                     "algorithmic_bytes": nbytes},
        "mfma": {"chunk_run": fr["chunk_run"],
                 "flops_per_step_at_run_chunk": T * H * flops_per_head_token(fr["chunk_run"]),
                 "frac_of_bf16_peak": fr["mfma_frac_at_run_chunk"],
                 "flops_per_step_F64": T * H * flops_per_head_token(64),
                 "frac_of_bf16_peak_F64": fr["mfma_frac_F64"],
                 "target_frac": MFMA_TARGET,
                 "gap_to_target": round(MFMA_TARGET - fr["mfma_frac_at_run_chunk"], 4),
                 "note": "HBM-bound: at the HBM roofline %MFMA would be ~0.27 at the run chunk "
                         "(0.35 at F(64)), below the 0.40 target"},
        "kernel_source_hash": src_hash,
    }
    if decode_out is not None:
        out["decode"] = decode_out
    # ---------------- prefix snapshots every 512 tokens (same workload) ----------------
    if not args.no_extra:
        snap_cu, n_snap = kda.snapshot_index(None, T, 512)
        snap = torch.empty((n_snap, H, D, D), dtype=torch.float32, device=dev)

        def sstep(i):
            d = sets[i % 2]
            kda.kda_chunk_fwd_snap(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                   interval=512, o=o, h_T=hT, snap=snap, snap_cu=snap_cu,
                                   n_snap=n_snap)

        _, sms = time_launches(sstep, args.steps, args.warmup, stream)
        savg = sum(sms) / len(sms)
        smed = median(sms)
        sbytes = nbytes + n_snap * H * D * D * 4
        # the overhead compares medians: one stalled launch among a few
        # hundred moves a mean by tens of percent
        out["snapshots"] = {"interval": 512, "entries": n_snap, "kernel_ms": round(savg, 5),
                            "kernel_ms_median": round(smed, 5),
                            "overhead_vs_plain": round(smed / median(ms) - 1.0, 4),
                            "algorithmic_bytes": sbytes,
                            "hbm_frac": round(sbytes / (smed * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}
        del snap
    del sets, o, hT
    torch.cuda.empty_cache()

    # ---------------- speculative verify + replay, 256 requests ----------------
    if not args.no_extra and not args.no_decode:
        out["verify_replay"] = verify_replay(torch, kda, kda_inputs, dev, stream, args.steps,
                                             args.warmup)

    if not args.no_extra:
        out["backward"] = backward(torch, kda, kda_inputs, dev, stream, args.steps, args.warmup,
                                   avg_ms)
        out["layer_elementwise"] = layer_elementwise(
            torch, kda, kda_inputs, dev, stream, args.steps, args.warmup, avg_ms,
            out["decode"]["ms_per_step"] if "decode" in out else None)

    if "verify_replay" in out and "decode" in out:
        vr = out["verify_replay"]
        vr["vs_7_decode_steps"] = round(
            7 * out["decode"]["ms_per_step"] / (vr["verify_ms"] + vr["replay_ms"]), 2)

    # measured streaming ceiling: fractions against it beside the 8 TB/s peak
    cbw = copy_bandwidth(torch, dev, stream)
    out["copy_GBps"] = cbw
    out["roofline"]["frac_of_copy"] = round(achieved / cbw, 4)
    if "decode" in out:
        out["decode"]["roofline"]["frac_of_copy"] = round(
            out["decode"]["roofline"]["achieved"] / cbw, 4)

    # every other workload, each with the CPU oracle beside it
    cpu = not args.no_cpu_baseline
    if not args.no_extra:
        extra = [extra_prefill(torch, kda, kda_inputs, dev, stream, 0, args.steps, args.warmup,
                               cpu=cpu),
                 extra_prefill(torch, kda, kda_inputs, dev, stream, 3, args.steps, args.warmup,
                               cpu=cpu)]
        out["context_parallel"] = context_parallel(torch, kda, kda_inputs, dev, stream,
                                                   min(args.steps, 5), 1)
        if not args.skip_long:
            extra.append(extra_prefill(torch, kda, kda_inputs, dev, stream, 4,
                                       args.long_steps, 1, cpu=cpu))
        out["other_workloads"] = extra

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst

    if cpu:
        out["cpu_baseline"] = cpu_baseline(T, H)
        # the oracle beside the other rows, on bounded samples
        if "decode" in out:
            out["decode"]["cpu_oracle"] = cpu_oracle_rows("decode")
        if "backward" in out:
            out["backward"]["cpu_oracle"] = cpu_oracle_rows("backward")
        if "layer_elementwise" in out:
            out["layer_elementwise"]["cpu_oracle"] = cpu_oracle_rows("layer")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
