"""MI355X (gfx950) Kimi Delta Attention: Python binding of libkda.so.

Thin ctypes marshalling over the C ABI in ``include/kda.h``; every step of
the computation runs in the HIP kernels of ``csrc/``.  PyTorch supplies the
device memory and the current stream only.  There is no fallback: if the
library is not built, or a tensor is not on a ROCm device, the call raises.

Functions (same names as the C entry points):

* ``kda_chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, ...)``
  -> ``(o, h_T)``  chunkwise prefill over packed sequences;
* ``kda_chunk_fwd_snap(..., interval=512)`` -> ``(o, h_T, snap, snap_cu)``
  the same, plus prefix snapshots of the state (``snapshot_index`` gives
  their layout);
* ``kda_decode_step(q, k, v, log_alpha, beta, S)`` -> ``o``  one recurrent
  step, ``S`` updated in place;
* ``kda_decode_multi(q, k, v, log_alpha, beta, S, n_tok)`` -> ``o``  up to K
  steps per sequence in one pass over the states (speculative verify /
  replay);
* ``kda_segment_summary`` -> ``(M, B)`` and ``kda_segment_scan`` -> ``(S_in,
  S_final)``  the affine summaries of sequence segments and the scan that
  chains them (context parallelism);
* ``kda_chunk_bwd`` -> ``(dq, dk, dv, dlog_alpha, dbeta, dh0)``  the
  backward (training) pass of the chunkwise forward, and
  ``kda_chunk_bwd_noalloc``, the same without a workspace (for callers that
  cannot allocate: the tables live in the library's static device scratch);
* ``kda_prologue`` and ``kda_epilogue``  the elementwise work of a KDA layer
  around the core (short convolution, Swish, norms, gates);
* ``kda_chunk_fwd_workspace_size``, ``kda_status_str``, ``kda_abi_version``.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
HEAD_DIM = 128

_lib = None


class KDAError(RuntimeError):
    """A nonzero kda_status from the library."""

    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


def lib():
    """The loaded libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m gated_delta_rule_27_amd.build` "
                "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.kda_abi_version.restype = ctypes.c_int
        L.kda_abi_version.argtypes = []
        L.kda_status_str.restype = ctypes.c_char_p
        L.kda_status_str.argtypes = [ctypes.c_int]
        L.kda_chunk_fwd_workspace_size.restype = sz
        L.kda_chunk_fwd_workspace_size.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int]
        L.kda_chunk_fwd.restype = ctypes.c_int
        L.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                    ctypes.c_int, vp, vp, vp, sz, vp]
        L.kda_chunk_fwd_ex.restype = ctypes.c_int
        L.kda_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                       ctypes.c_int, vp, vp, vp, sz, i32, i32, vp]
        L.kda_chunk_fwd_snap.restype = ctypes.c_int
        L.kda_chunk_fwd_snap.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                         ctypes.c_int, vp, vp, i32, vp, i64, vp, vp, sz, vp]
        L.kda_decode_step.restype = ctypes.c_int
        L.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                      ctypes.c_int, vp, vp]
        L.kda_decode_multi.restype = ctypes.c_int
        L.kda_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                       ctypes.c_int, i32, vp, vp]
        L.kda_segment_summary.restype = ctypes.c_int
        L.kda_segment_summary.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                          ctypes.c_int, vp, vp, vp, sz, vp]
        L.kda_segment_scan.restype = ctypes.c_int
        L.kda_segment_scan.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
        L.kda_prologue.restype = ctypes.c_int
        L.kda_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                   ctypes.c_int, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp,
                                   vp]
        L.kda_epilogue.restype = ctypes.c_int
        L.kda_epilogue.argtypes = [vp, vp, vp, i64, i32, i32, ctypes.c_int, ctypes.c_float,
                                   vp, vp]
        L.kda_chunk_bwd_workspace_size.restype = sz
        L.kda_chunk_bwd_workspace_size.argtypes = [i64, i32, i32, i32, i32, ctypes.c_int]
        L.kda_chunk_bwd.restype = ctypes.c_int
        L.kda_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                    ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.kda_chunk_bwd_noalloc.restype = ctypes.c_int
        L.kda_chunk_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                            i32, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp,
                                            vp]
        _lib = L
    return _lib


def kda_abi_version():
    return lib().kda_abi_version()


def kda_status_str(code):
    return lib().kda_status_str(int(code)).decode()


def kda_chunk_fwd_workspace_size(T_total, N, H, Dk=HEAD_DIM, Dv=HEAD_DIM, dtype=KDA_BF16):
    return lib().kda_chunk_fwd_workspace_size(int(T_total), int(N), int(H), int(Dk),
                                              int(Dv), int(dtype))


def _check(code):
    if code != 0:
        raise KDAError(code, kda_status_str(code))


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, name, dtype=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return t


def _tensors(**named):
    """Every argument given must be a torch.Tensor (None = not given)."""
    torch = _torch()
    for name, t in named.items():
        if t is not None and not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")


def _shape(t, name, shape):
    """Shape check of a caller-supplied tensor (None = not given).  The C ABI
    receives bare pointers, so a buffer that is too small would be written
    past its end: every output and optional input is checked here, before
    any device work."""
    shape = tuple(int(x) for x in shape)
    if t is not None and tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {shape} (got {tuple(t.shape)})")


def _shape_at_least(t, name, n0, rest):
    """A buffer of at least n0 entries of shape `rest` (None = not given):
    the C call writes entries below n0 only."""
    rest = tuple(int(x) for x in rest)
    if t is not None and (t.dim() != 1 + len(rest) or tuple(t.shape[1:]) != rest
                          or t.shape[0] < int(n0)):
        raise ValueError(f"{name} must have shape (>= {int(n0)},) + {rest} "
                         f"(got {tuple(t.shape)})")


def _same_device(dev, **named):
    for name, t in named.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} must be on {dev} like q (got {t.device})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _prefill_shapes(q, k, v, log_alpha, beta, h0, cu_seqlens, need_v=True):
    """Shape checks shared by the prefill-family calls; returns (T, H, Dk,
    Dv, N)."""
    _tensors(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, h0=h0, cu_seqlens=cu_seqlens)
    if q is None or k is None or log_alpha is None or beta is None or (need_v and v is None):
        raise TypeError("q, k, log_alpha, beta (and v) are required tensors")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, D]")
    T, H, Dk = q.shape
    Dv = v.shape[-1] if v is not None else Dk
    if k.shape != q.shape or log_alpha.shape != q.shape or tuple(beta.shape) != (T, H) \
            or (v is not None and (v.dim() != 3 or tuple(v.shape[:2]) != (T, H))):
        raise ValueError("inconsistent shapes")
    N = 1
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
        N = cu_seqlens.numel() - 1
    _shape(h0, "h0", (N, H, Dk, Dv))
    return T, H, Dk, Dv, N


def _prefill_devices(q, k, v, log_alpha, beta, h0, cu_seqlens):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta)):
        _dev(t, name, q.dtype)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(h0, "h0", torch.float32)
    _same_device(q.device, k=k, v=v, log_alpha=log_alpha, beta=beta, h0=h0,
                 cu_seqlens=cu_seqlens)


def kda_chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, chunk=0,
                  dv_split=0, o=None, h_T=None, store_state=True):
    """Chunkwise KDA prefill.

    q, k, log_alpha: [T, H, 128]; v: [T, H, 128]; beta: [T, H]; all bf16 or
    all fp32 on one device.  h0: [N, H, 128, 128] fp32 or None (zeros).
    cu_seqlens: int32 [N+1] device offsets or None (one sequence).
    Returns (o [T, H, 128] in the input dtype, h_T fp32 [N, H, 128, 128] or
    None if store_state is False).  `chunk` / `dv_split` override the
    library's tuning choice (0 = automatic).
    """
    torch = _torch()
    T, H, Dk, Dv, N = _prefill_shapes(q, k, v, log_alpha, beta, h0, cu_seqlens)
    _tensors(o=o, h_T=h_T)
    _shape(o, "o", (T, H, Dv))
    _shape(h_T, "h_T", (N, H, Dk, Dv))
    _prefill_devices(q, k, v, log_alpha, beta, h0, cu_seqlens)
    _dev(o, "o", q.dtype)
    _dev(h_T, "h_T", torch.float32)
    _same_device(q.device, o=o, h_T=h_T)
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty((T, H, Dv), dtype=q.dtype, device=q.device)
    if store_state and h_T is None:
        h_T = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if not store_state:
        h_T = None
    ws_bytes = kda_chunk_fwd_workspace_size(T, N, H, Dk, Dv, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    _check(lib().kda_chunk_fwd_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0), _ptr(cu_seqlens),
        N, T, H, Dk, Dv, dt, _ptr(o), _ptr(h_T), _ptr(ws), ws_bytes, int(chunk),
        int(dv_split), _stream(q.device)))
    return o, h_T


def snapshot_index(cu_seqlens, T_total, interval):
    """Layout of the prefix snapshots of kda_chunk_fwd_snap: returns
    (snap_cu, n_snap).  snap_cu is the int32 device tensor [N+1] with
    snap_cu[n] = sum over m < n of floor(len_m / interval) (None for one
    sequence, whose entries start at 0); sequence n's snapshot after
    j * interval tokens is entry snap_cu[n] + j - 1.  n_snap needs one
    device-to-host read when cu_seqlens is given."""
    torch = _torch()
    interval = int(interval)
    if interval <= 0:
        raise ValueError("interval must be positive")
    if cu_seqlens is None:
        return None, int(T_total) // interval
    cu = cu_seqlens.to(torch.int64)
    counts = (cu[1:] - cu[:-1]) // interval
    snap_cu = torch.zeros(cu.numel(), dtype=torch.int64, device=cu.device)
    snap_cu[1:] = torch.cumsum(counts, 0)
    return snap_cu.to(torch.int32), int(snap_cu[-1].item())


def kda_chunk_fwd_snap(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, interval,
                       o=None, h_T=None, snap=None, snap_cu=None, n_snap=None,
                       store_state=True):
    """kda_chunk_fwd that also writes the state of every sequence after each
    multiple of `interval` tokens (a multiple of 16) to `snap`
    [n_snap, H, 128, 128] fp32 (a longer buffer is allowed: entries at or
    past n_snap are never written), laid out as snapshot_index describes.
    Returns (o, h_T, snap, snap_cu)."""
    torch = _torch()
    T, H, Dk, Dv, N = _prefill_shapes(q, k, v, log_alpha, beta, h0, cu_seqlens)
    _tensors(o=o, h_T=h_T, snap=snap, snap_cu=snap_cu)
    _shape(o, "o", (T, H, Dv))
    _shape(h_T, "h_T", (N, H, Dk, Dv))
    if (snap_cu is None) != (n_snap is None) and N > 1:
        raise ValueError("give snap_cu and n_snap together (snapshot_index computes both)")
    if n_snap is not None:
        n_snap = int(n_snap)
        if n_snap < 0:
            raise ValueError("n_snap must be >= 0")
        _shape(snap_cu, "snap_cu", (N + 1,))
        _shape_at_least(snap, "snap", n_snap, (H, Dk, Dv))
    _prefill_devices(q, k, v, log_alpha, beta, h0, cu_seqlens)
    _dev(o, "o", q.dtype)
    _dev(h_T, "h_T", torch.float32)
    _dev(snap, "snap", torch.float32)
    _dev(snap_cu, "snap_cu", torch.int32)
    _same_device(q.device, o=o, h_T=h_T, snap=snap, snap_cu=snap_cu)
    dt = _dtype_code(q)
    if n_snap is None:
        snap_cu, n_snap = snapshot_index(cu_seqlens, T, interval)
        _shape_at_least(snap, "snap", n_snap, (H, Dk, Dv))
    if snap is None:
        snap = torch.empty((n_snap, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if o is None:
        o = torch.empty((T, H, Dv), dtype=q.dtype, device=q.device)
    if store_state and h_T is None:
        h_T = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    if not store_state:
        h_T = None
    ws_bytes = kda_chunk_fwd_workspace_size(T, N, H, Dk, Dv, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    _check(lib().kda_chunk_fwd_snap(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0), _ptr(cu_seqlens),
        N, T, H, Dk, Dv, dt, _ptr(o), _ptr(h_T), int(interval), _ptr(snap_cu), int(n_snap),
        _ptr(snap), _ptr(ws), ws_bytes, _stream(q.device)))
    return o, h_T, snap, snap_cu


def kda_decode_step(q, k, v, log_alpha, beta, S, *, o=None):
    """One recurrent KDA step for B sequences; S [B, H, 128, 128] fp32 is
    updated in place.  q, k, log_alpha, v: [B, H, 128]; beta: [B, H].
    Returns o [B, H, 128] in the input dtype."""
    torch = _torch()
    _tensors(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, S=S, o=o)
    if q.dim() != 3:
        raise ValueError("q must be [B, H, D]")
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.dim() != 3 \
            or tuple(v.shape[:2]) != (B, H) or tuple(beta.shape) != (B, H):
        raise ValueError("inconsistent shapes")
    _shape(S, "S", (B, H, Dk, Dv))
    _shape(o, "o", (B, H, Dv))
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta)):
        _dev(t, name, q.dtype)
    _dev(S, "S", torch.float32)
    _dev(o, "o", q.dtype)
    _same_device(q.device, k=k, v=v, log_alpha=log_alpha, beta=beta, S=S, o=o)
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    _check(lib().kda_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), B, H, Dk, Dv, dt,
        _ptr(o), _stream(q.device)))
    return o


def kda_segment_summary(q, k, v, log_alpha, beta, cu_seqlens=None, *, want_M=True,
                        want_B=True):
    """Affine summaries S_out = M S_in + B of the segments given by
    cu_seqlens (packed as for kda_chunk_fwd).  Returns (M, B), each
    [N, H, 128, 128] fp32 or None when not asked for."""
    torch = _torch()
    if not want_B:
        v = None
    T, H, Dk, _, N = _prefill_shapes(q, k, v, log_alpha, beta, None, cu_seqlens,
                                     need_v=want_B)
    if v is not None and v.shape[-1] != Dk:
        raise ValueError("v must be [T, H, 128]")
    _prefill_devices(q, k, v, log_alpha, beta, None, cu_seqlens)
    dt = _dtype_code(q)
    M = torch.empty((N, H, Dk, Dk), dtype=torch.float32, device=q.device) if want_M else None
    B = torch.empty((N, H, Dk, Dk), dtype=torch.float32, device=q.device) if want_B else None
    ws_bytes = kda_chunk_fwd_workspace_size(T, N, H, Dk, Dk, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    _check(lib().kda_segment_summary(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(cu_seqlens), N, T, H,
        Dk, Dk, dt, _ptr(M), _ptr(B), _ptr(ws), ws_bytes, _stream(q.device)))
    return M, B


def kda_segment_scan(M, B, h0=None):
    """States entering R consecutive segments: S_in[0] = h0 (None = 0),
    S_in[r+1] = M[r] S_in[r] + B[r].  M, B: [R, H, 128, 128] fp32; h0:
    [H, 128, 128] or [1, H, 128, 128].  Returns (S_in [R, H, 128, 128],
    S_final [H, 128, 128])."""
    torch = _torch()
    _tensors(M=M, B=B, h0=h0)
    if M.dim() != 4:
        raise ValueError("M must be [R, H, 128, 128]")
    R, H, Dk, Dv = M.shape
    _shape(B, "B", (R, H, Dk, Dv))
    if h0 is not None:
        if h0.numel() != H * Dk * Dv:
            raise ValueError(f"h0 must be [H, Dk, Dv] or [1, H, Dk, Dv] (got {tuple(h0.shape)})")
        h0 = h0.reshape(H, Dk, Dv)
    _dev(M, "M", torch.float32)
    _dev(B, "B", torch.float32)
    _dev(h0, "h0", torch.float32)
    _same_device(M.device, B=B, h0=h0)
    S_in = torch.empty_like(M)
    S_final = torch.empty((H, Dk, Dv), dtype=torch.float32, device=M.device)
    _check(lib().kda_segment_scan(_ptr(M), _ptr(B), _ptr(h0), R, H, Dk, Dv, _ptr(S_in),
                                  _ptr(S_final), _stream(M.device)))
    return S_in, S_final


def kda_chunk_bwd_workspace_size(T_total, N, H, Dk=HEAD_DIM, Dv=HEAD_DIM, dtype=KDA_BF16):
    return lib().kda_chunk_bwd_workspace_size(int(T_total), int(N), int(H), int(Dk), int(Dv),
                                              int(dtype))


def kda_chunk_bwd(q, k, v, log_alpha, beta, do, h0=None, cu_seqlens=None, dhT=None, *,
                  want_dh0=True, workspace=None):
    """Backward of kda_chunk_fwd for the loss sum(do * o) + sum(dhT * h_T).

    Inputs as kda_chunk_fwd plus do [T, H, 128] (input dtype) and dhT
    [N, H, 128, 128] fp32 or None.  Returns (dq, dk, dv, dlog_alpha, dbeta,
    dh0 or None); token gradients in the input dtype, dh0 fp32."""
    torch = _torch()
    T, H, Dk, Dv, N = _prefill_shapes(q, k, v, log_alpha, beta, h0, cu_seqlens)
    _tensors(do=do, dhT=dhT, workspace=workspace)
    _shape(do, "do", (T, H, Dv))
    _shape(dhT, "dhT", (N, H, Dk, Dv))
    _prefill_devices(q, k, v, log_alpha, beta, h0, cu_seqlens)
    _dev(do, "do", q.dtype)
    _dev(dhT, "dhT", torch.float32)
    _dev(workspace, "workspace")
    _same_device(q.device, do=do, dhT=dhT, workspace=workspace)
    dt = _dtype_code(q)
    dq, dk, dv, dg = (torch.empty_like(x) for x in (q, k, v, log_alpha))
    db = torch.empty_like(beta)
    dh0 = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device) if want_dh0 else None
    ws_bytes = kda_chunk_bwd_workspace_size(T, N, H, Dk, Dv, dt)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check(lib().kda_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), N,
        T, H, Dk, Dv, dt, _ptr(do), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db),
        _ptr(dh0), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q.device)))
    return dq, dk, dv, dg, db, dh0


# KDA_BWD_NOALLOC_MAX_BYTES of include/kda.h: the largest backward workspace
# kda_chunk_bwd_noalloc serves from the library's own device scratch
BWD_NOALLOC_MAX_BYTES = 256 << 20


def kda_chunk_bwd_noalloc(q, k, v, log_alpha, beta, do, h0=None, cu_seqlens=None, dhT=None, *,
                          want_dh0=True, grads=None):
    """kda_chunk_bwd without a workspace argument: the per-chunk tables live
    in the library's static device scratch (at most BWD_NOALLOC_MAX_BYTES of
    workspace, i.e. kda_chunk_bwd_workspace_size must not exceed it).  The C
    call allocates nothing; `grads` may supply the six output tensors
    (dq, dk, dv, dlog_alpha, dbeta, dh0-or-None) so that this function
    allocates nothing either.  Calls that overlap on one GPU share the
    scratch: keep them on one stream.  Returns the six gradients."""
    torch = _torch()
    T, H, Dk, Dv, N = _prefill_shapes(q, k, v, log_alpha, beta, h0, cu_seqlens)
    _tensors(do=do, dhT=dhT)
    _shape(do, "do", (T, H, Dv))
    _shape(dhT, "dhT", (N, H, Dk, Dv))
    if grads is not None:
        if len(grads) != 6:
            raise ValueError("grads must be (dq, dk, dv, dlog_alpha, dbeta, dh0 or None)")
        _tensors(**dict(zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0"), grads)))
        for name, t, shape in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0"), grads,
                                  ((T, H, Dk), (T, H, Dk), (T, H, Dv), (T, H, Dk), (T, H),
                                   (N, H, Dk, Dv))):
            _shape(t, name, shape)
    _prefill_devices(q, k, v, log_alpha, beta, h0, cu_seqlens)
    _dev(do, "do", q.dtype)
    _dev(dhT, "dhT", torch.float32)
    _same_device(q.device, do=do, dhT=dhT)
    dt = _dtype_code(q)
    if grads is None:
        dq, dk, dv, dg = (torch.empty_like(x) for x in (q, k, v, log_alpha))
        db = torch.empty_like(beta)
        dh0 = (torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
               if want_dh0 else None)
    else:
        dq, dk, dv, dg, db, dh0 = grads
        for name, t in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta"), (dq, dk, dv, dg, db)):
            _dev(t, name, q.dtype)
        _dev(dh0, "dh0", torch.float32)
        _same_device(q.device, dq=dq, dk=dk, dv=dv, dlog_alpha=dg, dbeta=db, dh0=dh0)
    _check(lib().kda_chunk_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), N,
        T, H, Dk, Dv, dt, _ptr(do), _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db),
        _ptr(dh0), _stream(q.device)))
    return dq, dk, dv, dg, db, dh0


def kda_prologue(xq, xk, xv, a_raw, b_raw, conv_w, a_bias, cu_seqlens=None, conv_state=None,
                 *, l2_eps=1e-6, store_state=True, state_out=None):
    """Prologue of a KDA layer: Swish(short conv) for q, k, v (q, k then
    L2-normalised per head), log_alpha = -5 sigmoid(a_raw + a_bias), beta =
    sigmoid(b_raw), and the new convolution history.

    xq, xk, xv, a_raw: [T, H, 128]; b_raw: [T, H] (bf16 or fp32, one dtype);
    conv_w: [3, H, 128, 4] fp32; a_bias: [H, 128] fp32; conv_state:
    [N, 3, 3, H, 128] in the input dtype or None (zero history).  Returns
    (q, k, v, log_alpha, beta, conv_state_out or None)."""
    torch = _torch()
    _tensors(xq=xq, xk=xk, xv=xv, a_raw=a_raw, b_raw=b_raw, conv_w=conv_w, a_bias=a_bias,
             cu_seqlens=cu_seqlens, conv_state=conv_state, state_out=state_out)
    if xq.dim() != 3:
        raise ValueError("xq must be [T, H, D]")
    dt_t = xq.dtype
    T, H, D = xq.shape
    for name, t in (("xk", xk), ("xv", xv), ("a_raw", a_raw)):
        _shape(t, name, (T, H, D))
    _shape(b_raw, "b_raw", (T, H))
    _shape(conv_w, "conv_w", (3, H, D, 4))
    _shape(a_bias, "a_bias", (H, D))
    N = 1
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [N + 1] with N >= 1")
        N = cu_seqlens.numel() - 1
    _shape(conv_state, "conv_state", (N, 3, 3, H, D))
    _shape(state_out, "state_out", (N, 3, 3, H, D))
    for name, t in (("xq", xq), ("xk", xk), ("xv", xv), ("a_raw", a_raw), ("b_raw", b_raw)):
        _dev(t, name, dt_t)
    _dev(conv_w, "conv_w", torch.float32)
    _dev(a_bias, "a_bias", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(conv_state, "conv_state", dt_t)
    _dev(state_out, "state_out", dt_t)
    _same_device(xq.device, xk=xk, xv=xv, a_raw=a_raw, b_raw=b_raw, conv_w=conv_w,
                 a_bias=a_bias, cu_seqlens=cu_seqlens, conv_state=conv_state,
                 state_out=state_out)
    dt = _dtype_code(xq)
    q, k, v, la = (torch.empty_like(xq) for _ in range(4))
    beta = torch.empty_like(b_raw)
    so = None
    if store_state:
        so = state_out if state_out is not None else torch.empty(
            (N, 3, 3, H, D), dtype=dt_t, device=xq.device)
    _check(lib().kda_prologue(
        _ptr(xq), _ptr(xk), _ptr(xv), _ptr(a_raw), _ptr(b_raw), _ptr(conv_w), _ptr(a_bias),
        _ptr(cu_seqlens), N, T, H, D, dt, _ptr(conv_state), _ptr(so), float(l2_eps), _ptr(q),
        _ptr(k), _ptr(v), _ptr(la), _ptr(beta), _stream(xq.device)))
    return q, k, v, la, beta, so


def kda_epilogue(o, g, norm_w, *, eps=1e-5, y=None):
    """y = RMSNorm_head(o) * norm_w * sigmoid(g).  o, g: [T, H, 128]
    (bf16 or fp32); norm_w: [H, 128] fp32.  y may be o or g (in place)."""
    torch = _torch()
    _tensors(o=o, g=g, norm_w=norm_w, y=y)
    if o.dim() != 3:
        raise ValueError("o must be [T, H, D]")
    T, H, D = o.shape
    _shape(g, "g", (T, H, D))
    _shape(norm_w, "norm_w", (H, D))
    _shape(y, "y", (T, H, D))
    _dev(o, "o", o.dtype)
    _dev(g, "g", o.dtype)
    _dev(norm_w, "norm_w", torch.float32)
    _dev(y, "y", o.dtype)
    _same_device(o.device, g=g, norm_w=norm_w, y=y)
    if y is None:
        y = torch.empty_like(o)
    _check(lib().kda_epilogue(_ptr(o), _ptr(g), _ptr(norm_w), T, H, D, _dtype_code(o),
                              float(eps), _ptr(y), _stream(o.device)))
    return y


def kda_decode_multi(q, k, v, log_alpha, beta, S, n_tok=None, *, update_state=True, o=None):
    """Up to K recurrent KDA steps for B sequences in one pass over their
    states.  q, k, log_alpha, v: [B, K, H, 128]; beta: [B, K, H]; S
    [B, H, 128, 128] fp32, written back in place iff update_state; n_tok:
    int32 [B] device (tokens applied per sequence, clamped to [0, K]) or
    None (all K).  Returns o [B, K, H, 128] (rows past n_tok[b] untouched)."""
    torch = _torch()
    _tensors(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, S=S, n_tok=n_tok, o=o)
    if q.dim() != 4:
        raise ValueError("q must be [B, K, H, D]")
    B, K, H, Dk = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.dim() != 4 \
            or tuple(v.shape[:3]) != (B, K, H) or tuple(beta.shape) != (B, K, H):
        raise ValueError("inconsistent shapes")
    _shape(S, "S", (B, H, Dk, Dv))
    _shape(n_tok, "n_tok", (B,))
    _shape(o, "o", (B, K, H, Dv))
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta)):
        _dev(t, name, q.dtype)
    _dev(S, "S", torch.float32)
    _dev(n_tok, "n_tok", torch.int32)
    _dev(o, "o", q.dtype)
    _same_device(q.device, k=k, v=v, log_alpha=log_alpha, beta=beta, S=S, n_tok=n_tok, o=o)
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty((B, K, H, Dv), dtype=q.dtype, device=q.device)
    _check(lib().kda_decode_multi(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(n_tok),
        B, K, H, Dk, Dv, dt, 1 if update_state else 0, _ptr(o), _stream(q.device)))
    return o


__all__ = ["kda_chunk_fwd", "kda_chunk_fwd_snap", "snapshot_index", "kda_decode_step",
           "kda_decode_multi", "kda_segment_summary", "kda_segment_scan", "kda_prologue",
           "kda_epilogue", "kda_chunk_bwd", "kda_chunk_bwd_workspace_size",
           "kda_chunk_bwd_noalloc", "BWD_NOALLOC_MAX_BYTES",
           "kda_chunk_fwd_workspace_size", "kda_status_str", "kda_abi_version", "KDAError",
           "lib", "LIB_PATH"]
