"""CPU checks of bench.py's work accounting.

The throughput and roofline figures divide by algorithmic work per unit:
1282 B per (token, head) of a bf16 prefill (q, k, v, log alpha and o at
256 B each, beta 2 B) plus 64 KiB per (sequence, head) for each fp32
state moved; 132,354 B per (sequence, head) of a decode step (the state
read and written, 128 x 128 fp32 each way, plus the token's vectors); and
F(C) = 6 d^2 + d (5 C + 3) + C^2 / 3 flops per (token, head) at chunk
length C.  These tests evaluate bench.py's helpers at the workload sizes
against the same figures computed here by hand, and check that the
committed HBM-traffic summary of the prefill kernel parses and stays
close to the algorithmic bytes."""
import os

import pytest

import bench


def test_prefill_bytes_per_unit():
    assert bench.prefill_bytes(1, 1, 0) == 1282
    assert bench.prefill_bytes(1, 1, 0, esize=4) == 2564
    assert bench.prefill_bytes(0, 1, 1) == 128 * 128 * 4
    assert bench.prefill_bytes(0, 1, 1, h0=True) == 2 * 128 * 128 * 4


@pytest.mark.parametrize("T, H, N, expected", [
    (4096, 96, 1, 510_394_368),            # one 4096-token sequence, 96 heads
    (1_048_576, 96, 1, 129_056_636_928),   # one 1,048,576-token sequence
    (128, 2, 1, 128 * 2 * 1282 + 2 * 65536),
])
def test_prefill_bytes_at_workload_sizes(T, H, N, expected):
    assert bench.prefill_bytes(T, H, N) == expected


def test_decode_bytes():
    assert bench.decode_bytes(1, 1) == 132_354
    assert bench.decode_bytes(256, 96) == 3_252_731_904


def test_flops_per_head_token():
    assert round(bench.flops_per_head_token(64)) == 141_013
    assert round(bench.flops_per_head_token(16)) == 109_013
    # with no chunk-local work left: the three state products (6 d^2) and
    # the 3 d of elementwise terms
    assert bench.flops_per_head_token(0) == 6 * 128 * 128 + 3 * 128


def test_mfma_fracs():
    r = bench.mfma_fracs(4096, 96, 1.0)   # one millisecond
    peak = bench.BF16_PEAK_TFLOPS * 1e12 * 1e-3
    assert r["chunk_run"] == bench.RUN_CHUNK
    assert r["mfma_frac_F64"] == round(4096 * 96 * bench.flops_per_head_token(64) / peak, 4)
    assert r["mfma_frac_at_run_chunk"] == round(
        4096 * 96 * bench.flops_per_head_token(bench.RUN_CHUNK) / peak, 4)


def test_committed_prefill_traffic_summary():
    path = os.path.join(bench.ROOT, "profiles", "chunk_fwd_T4096_H96_bf16_traffic.txt")
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    measured = float(vals["hbm_bytes_per_launch"])
    reads = float(vals["fetch_kib"]) * 1024 * float(vals["read_scale"])
    writes = float(vals["write_kib"]) * 1024 * float(vals["write_scale"])
    assert abs(reads + writes - measured) <= 1e-4 * measured   # scales printed to 4 places
    # no re-reads beyond a few percent of the algorithmic bytes
    assert 1.0 <= measured / bench.prefill_bytes(4096, 96, 1) < 1.05
    # the o and h_T writes: 100.7 MB + 6.3 MB
    assert abs(writes - (4096 * 96 * 256 + 96 * 65536)) < 0.01 * writes
