"""Helpers for the GPU parity tests: run the HIP path through the C ABI
binding, run the fp64 oracle on exactly the same (widened) input bytes, and
compare.  Test infrastructure only."""
import sys

import numpy as np
import pytest
import torch

import kda_inputs
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def case(msg):
    """Name the case before any GPU work, so a failing run says which."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    import gated_delta_rule_27_amd as kda
    kda.lib()  # raises if the HIP library is missing: no fallback
    return kda


def nerr(x, ref):
    """Normwise error max|x - ref| / max|ref| (per tensor)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(x).max())
    return float(np.abs(x - ref).max() / den)


def elem_err(x, ref, floor=1e-3):
    """Elementwise relative error with a floor of floor * max|ref|."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    f = floor * max(np.abs(ref).max(), 1e-300)
    return float((np.abs(x - ref) / np.maximum(np.abs(ref), f)).max())


def np_(t):
    return kda_inputs.to_numpy(t)


def oracle_prefill(d):
    """fp64 oracle on the inputs of a prefill dict (device or host tensors)."""
    cu = d["cu_seqlens"]
    cu_np = None if cu is None else cu.cpu().numpy().astype(np.int64)
    return oracle.fwd(np_(d["q"]), np_(d["k"]), np_(d["v"]), np_(d["log_alpha"]),
                      np_(d["beta"]), h0=np_(d["h0"]), cu_seqlens=cu_np)


def gpu_prefill(kda, d, chunk=0, split=0):
    o, hT = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], h0=d["h0"],
                              cu_seqlens=d["cu_seqlens"], chunk=chunk, dv_split=split)
    torch.cuda.synchronize()
    return o, hT


def check(name, got, ref, tol):
    e = nerr(got, ref)
    print(f"    {name}: normwise err {e:.3e} (tol {tol:.0e}), elementwise {elem_err(got, ref):.3e}",
          flush=True)
    assert np.isfinite(np.asarray(got, dtype=np.float64)).all(), f"{name}: non-finite output"
    assert e <= tol, f"{name}: normwise error {e:.3e} > {tol:.0e}"
    return e
