"""CPU oracle for Kimi Delta Attention (KDA) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports, links or calls it.

The arithmetic lives in the C library ``libkda_oracle.so`` (``kda_oracle.c``):
the token-by-token recurrence

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t,

from "Kimi K3 Architecture Explained" (Analytics Vidhya), Step 3, and the
KDA card of "An infra-oriented diagram of Kimi K3".  This module only
marshals NumPy arrays into it.

Inputs may be any float dtype (bfloat16 values arrive already widened to
float32 by the caller, which is exact); they are converted to float64 (the
parity reference, ``precision="f64"``) or float32 (the timed CPU baseline,
``precision="f32"``).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def load(path):
    """Load an oracle library from `path` and declare its signatures."""
    L = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    for sfx in ("f64", "f32"):
        f = getattr(L, "kda_oracle_fwd_" + sfx)
        f.restype = ctypes.c_int
        f.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                      vp, vp, i32, i32]
        d = getattr(L, "kda_oracle_decode_" + sfx)
        d.restype = ctypes.c_int
        d.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32]
    return L


def lib():
    """Load the oracle library, compiling it first if it is not built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = load(_build.LIB)
    return _LIB


def default_threads():
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _arr(x, dt):
    return np.ascontiguousarray(np.asarray(x), dtype=dt)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, precision="f64",
        nthreads=None, dv_block=0, store_state=True, library=None):
    """Prefill over packed sequences.

    q, k, log_alpha: [T, H, Dk]; v: [T, H, Dv]; beta: [T, H];
    h0: [N, H, Dk, Dv] or None (zeros); cu_seqlens: [N+1] offsets or None
    (one sequence).  Returns (o [T, H, Dv], h_T [N, H, Dk, Dv] or None).
    """
    dt = np.float64 if precision == "f64" else np.float32
    q, k, v = _arr(q, dt), _arr(k, dt), _arr(v, dt)
    g, b = _arr(log_alpha, dt), _arr(beta, dt)
    T, H, Dk = q.shape
    Dv = v.shape[2]
    if k.shape != (T, H, Dk) or g.shape != (T, H, Dk) or v.shape[:2] != (T, H) \
            or b.shape != (T, H):
        raise ValueError("inconsistent input shapes")
    if cu_seqlens is None:
        cu = None
        N = 1
    else:
        cu = _arr(cu_seqlens, np.int64)
        N = cu.shape[0] - 1
    if h0 is not None:
        h0 = _arr(h0, dt)
        if h0.shape != (N, H, Dk, Dv):
            raise ValueError("h0 must be [N, H, Dk, Dv]")
    o = np.zeros((T, H, Dv), dtype=dt)
    hT = np.zeros((N, H, Dk, Dv), dtype=dt) if store_state else None
    f = getattr(library or lib(), "kda_oracle_fwd_" + precision)
    rc = f(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(h0), _ptr(cu),
           N, T, H, Dk, Dv, _ptr(o), _ptr(hT), int(dv_block),
           int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (cu_seqlens?)")
    return o, hT


def decode(q, k, v, log_alpha, beta, S, precision="f64", nthreads=None,
           library=None):
    """One recurrent step for B sequences.

    q, k, log_alpha: [B, H, Dk]; v: [B, H, Dv]; beta: [B, H];
    S: [B, H, Dk, Dv] (not modified).  Returns (o [B, H, Dv], S_new).
    `library` (tests only) selects another build of the oracle, e.g. a
    deliberately broken copy used to check that the pins catch mistakes.
    """
    dt = np.float64 if precision == "f64" else np.float32
    q, k, v = _arr(q, dt), _arr(k, dt), _arr(v, dt)
    g, b = _arr(log_alpha, dt), _arr(beta, dt)
    S = np.array(S, dtype=dt, copy=True, order="C")
    B, H, Dk = q.shape
    Dv = v.shape[2]
    if S.shape != (B, H, Dk, Dv) or b.shape != (B, H):
        raise ValueError("inconsistent input shapes")
    o = np.zeros((B, H, Dv), dtype=dt)
    f = getattr(library or lib(), "kda_oracle_decode_" + precision)
    rc = f(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(S), B, H, Dk, Dv,
           _ptr(o), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, S
