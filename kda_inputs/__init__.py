"""Seeded synthetic inputs for the KDA workloads.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random numbers and shapes them into the workloads' distributions; it
holds none of the KDA recurrence's arithmetic (no decay, no delta update, no
read-out), so neither the oracle nor the HIP path depends on the other
through it.

Input distributions (the K3 KDA shape: 96 heads, d_k = d_v = 128; "An
infra-oriented diagram of Kimi K3", KDA card, and "From GPT-2 to Kimi K3",
ch. 5, "K3's lower-bounded decay"):

* q, k ~ N(0, 1) per element, then L2-normalised over the head dimension in
  fp32 (the pages normalise queries and keys before the recurrence), then
  rounded to the storage dtype (round-to-nearest-even for bf16);
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1)) per (token, head), in (0, 1);
* log_alpha = -5 * sigmoid(N(mu, 1)) per (token, head, key channel), in
  (-5, 0) -- the K3 lower-bounded log-decay.  mu = 0 is the workloads'
  distribution; mu = -4 or -8 gives the slow-decay stress variants;
* h0 (per-document initial state) and the decode state S ~ N(0, 0.02) fp32
  (0.02 is the standard deviation).

Inputs of the layer prologue / epilogue (the outputs of the layer's
projections, which are plain GEMMs outside this path): x_q, x_k, x_v, the
decay logits a and the write logits b ~ N(0, 1); the width-4 convolution
taps ~ N(0, 0.5^2) (so a tap sum of unit inputs has unit variance); the
decay bias ~ N(0, 1); a cached convolution history ~ N(0, 1); the core's
read-out o and the gate logits g ~ N(0, 1); the RMSNorm weight 1 + N(0, 0.1^2).

Every tensor has its own generator, seeded from (seed, tensor id), so the
shapes of one tensor never shift the stream of another.  Large tensors are
drawn in slabs of tokens to bound temporary memory; the slab order is fixed,
so the result is deterministic for a given device.
"""
import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}

# Tensor ids for the per-tensor generators.
_TID = {"q": 1, "k": 2, "v": 3, "log_alpha": 4, "beta": 5, "h0": 6, "S": 7,
        "xq": 11, "xk": 12, "xv": 13, "a_raw": 14, "b_raw": 15, "conv_w": 16, "a_bias": 17,
        "conv_state": 18, "o": 19, "g": 20, "norm_w": 21}

# The five workloads.  "chunk" is the chunk length fixed by a workload (only
# the tiny one fixes it).
CONFIGS = [
    dict(id=0, name="tiny_prefill_T128_H2_f32", kind="prefill", N=1, T=128, H=2,
         D=128, dtype="f32", chunk=16, h0=False),
    dict(id=1, name="prefill_T4096_H96_bf16", kind="prefill", N=1, T=4096, H=96,
         D=128, dtype="bf16", chunk=None, h0=False),
    dict(id=2, name="decode_B256_H96_bf16", kind="decode", B=256, H=96, D=128,
         dtype="bf16", state_std=0.02),
    dict(id=3, name="varlen_prefill_16docs_H96_bf16", kind="prefill", N=16,
         len_lo=512, len_hi=8192, H=96, D=128, dtype="bf16", chunk=None,
         h0=True, h0_std=0.02),
    dict(id=4, name="prefill_T1048576_H96_bf16", kind="prefill", N=1,
         T=1048576, H=96, D=128, dtype="bf16", chunk=None, h0=False),
]

_SLAB = 1 << 16  # tokens per generation slab


def _gen(device, seed, tid):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 100 + _TID[tid])
    return g


def _normal(shape, gen, device, mean=0.0, std=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x


def _fill_tokens(out, gen, device, kind, mu=0.0):
    """Fill out[T, ...] slab by slab with the distribution `kind`."""
    T = out.shape[0]
    for t0 in range(0, T, _SLAB):
        t1 = min(T, t0 + _SLAB)
        x = _normal((t1 - t0,) + tuple(out.shape[1:]), gen, device)
        if kind == "unit":          # L2-normalised over the last dimension
            x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        elif kind == "sigmoid":     # beta
            x = torch.sigmoid(x)
        elif kind == "logdecay":    # log alpha in (-5, 0)
            if mu != 0.0:
                x.add_(mu)
            x = -5.0 * torch.sigmoid(x)
        out[t0:t1].copy_(x)
    return out


def seq_lengths_varlen(n_docs=16, lo=512, hi=8192, seed=1003):
    """Document lengths drawn uniformly from the integers [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    return rng.integers(lo, hi + 1, size=n_docs).astype(np.int64)


def cu_from_lengths(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def prefill_inputs(T, H, Dk=128, Dv=128, dtype="bf16", device="cpu", seed=0,
                   lengths=None, h0_std=None, decay_mu=0.0, zero_decay=False,
                   beta_const=None, unit_keys=True):
    """Packed prefill inputs.

    lengths: per-sequence lengths (sum must equal T) or None for one
    sequence.  Returns a dict of tensors on `device`: q, k, log_alpha
    [T, H, Dk]; v [T, H, Dv]; beta [T, H] (all `dtype`); cu_seqlens int32
    [N+1] (None for one sequence); h0 fp32 [N, H, Dk, Dv] or None.
    """
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    dev = torch.device(device)
    if lengths is not None:
        cu = cu_from_lengths(lengths)
        if int(cu[-1]) != T:
            raise ValueError("lengths must sum to T")
        N = len(lengths)
    else:
        cu, N = None, 1
    out = {}
    for name, D, kind in (("q", Dk, "unit" if unit_keys else "normal"),
                          ("k", Dk, "unit" if unit_keys else "normal"),
                          ("v", Dv, "normal")):
        t = torch.empty((T, H, D), dtype=dt, device=dev)
        out[name] = _fill_tokens(t, _gen(dev, seed, name), dev, kind)
    g = torch.empty((T, H, Dk), dtype=dt, device=dev)
    if zero_decay:
        g.zero_()
    else:
        _fill_tokens(g, _gen(dev, seed, "log_alpha"), dev, "logdecay", decay_mu)
    out["log_alpha"] = g
    b = torch.empty((T, H), dtype=dt, device=dev)
    if beta_const is not None:
        b.fill_(float(beta_const))
    else:
        _fill_tokens(b, _gen(dev, seed, "beta"), dev, "sigmoid")
    out["beta"] = b
    out["cu_seqlens"] = (torch.as_tensor(cu, dtype=torch.int32, device=dev)
                         if cu is not None else None)
    if h0_std is not None:
        out["h0"] = _normal((N, H, Dk, Dv), _gen(dev, seed, "h0"), dev,
                            std=float(h0_std))
    else:
        out["h0"] = None
    out["N"] = N
    return out


def decode_inputs(B, H, Dk=128, Dv=128, dtype="bf16", device="cpu", seed=0,
                  state_std=0.02, decay_mu=0.0):
    """One-token decode inputs for B sequences: q, k, log_alpha [B, H, Dk],
    v [B, H, Dv], beta [B, H] (dtype) and the fp32 state S [B, H, Dk, Dv]."""
    d = prefill_inputs(B, H, Dk, Dv, dtype, device, seed, decay_mu=decay_mu)
    dev = torch.device(device)
    S = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    gen = _gen(dev, seed, "S")
    for b0 in range(0, B, 16):
        b1 = min(B, b0 + 16)
        S[b0:b1].copy_(_normal((b1 - b0, H, Dk, Dv), gen, dev, std=state_std))
    return dict(q=d["q"], k=d["k"], v=d["v"], log_alpha=d["log_alpha"],
                beta=d["beta"], S=S)


def layer_inputs(T, H, D=128, dtype="bf16", device="cpu", seed=0, lengths=None,
                 conv_state=False):
    """Inputs of the prologue and epilogue of a KDA layer.

    Returns a dict: xq, xk, xv, a_raw [T, H, D] and b_raw [T, H] (dtype);
    conv_w [3, H, D, 4] and a_bias [H, D] (fp32); conv_state
    [N, 3, 3, H, D] (dtype) or None; cu_seqlens int32 [N + 1] or None; o and
    g [T, H, D] (dtype); norm_w [H, D] (fp32); N."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    dev = torch.device(device)
    if lengths is not None:
        cu = cu_from_lengths(lengths)
        if int(cu[-1]) != T:
            raise ValueError("lengths must sum to T")
        N = len(lengths)
    else:
        cu, N = None, 1
    out = {"N": N, "cu_seqlens": (torch.as_tensor(cu, dtype=torch.int32, device=dev)
                                  if cu is not None else None)}
    for name in ("xq", "xk", "xv", "a_raw", "o", "g"):
        t = torch.empty((T, H, D), dtype=dt, device=dev)
        out[name] = _fill_tokens(t, _gen(dev, seed, name), dev, "normal")
    b = torch.empty((T, H), dtype=dt, device=dev)
    out["b_raw"] = _fill_tokens(b, _gen(dev, seed, "b_raw"), dev, "normal")
    out["conv_w"] = _normal((3, H, D, 4), _gen(dev, seed, "conv_w"), dev, std=0.5)
    out["a_bias"] = _normal((H, D), _gen(dev, seed, "a_bias"), dev)
    out["norm_w"] = _normal((H, D), _gen(dev, seed, "norm_w"), dev, mean=1.0, std=0.1)
    out["conv_state"] = (_normal((N, 3, 3, H, D), _gen(dev, seed, "conv_state"), dev).to(dt)
                         if conv_state else None)
    return out


def config_inputs(cfg_id, device="cpu", seed=None):
    """The inputs of workload `cfg_id` (seed 1000 + id unless given)."""
    c = CONFIGS[cfg_id]
    s = 1000 + cfg_id if seed is None else seed
    if c["kind"] == "decode":
        return decode_inputs(c["B"], c["H"], c["D"], c["D"], c["dtype"], device, s,
                             state_std=c["state_std"])
    if c["id"] == 3:
        lengths = seq_lengths_varlen(c["N"], c["len_lo"], c["len_hi"])
        T = int(lengths.sum())
        return prefill_inputs(T, c["H"], c["D"], c["D"], c["dtype"], device, s,
                              lengths=lengths, h0_std=c["h0_std"])
    return prefill_inputs(c["T"], c["H"], c["D"], c["D"], c["dtype"], device, s)


def to_numpy(t):
    """Exact widening of a torch tensor to a NumPy float array (bf16 -> f32)."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()
