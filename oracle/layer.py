"""CPU oracle for the elementwise prologue and epilogue around the KDA core
-- TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle``: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import it).

Plain NumPy in float64, one function per step, composed in the order the
pages give for a KDA layer ("From GPT-2 to Kimi K3", ch. 6, "Where q, k, v,
alpha, and beta come from" and "A third gate: control what leaves the
module"; "Kimi K3 Architecture Explained", "Inside a KDA Layer"; "An
infra-oriented diagram of Kimi K3", the Kimi Delta Attention card):

prologue, per head and token, on the outputs of the input projections
(the projections themselves are plain GEMMs and not part of this path):
  q, k, v   = Swish(ShortConv_4(x_q | x_k | x_v)), then q, k L2-normalised
              per head;
  log alpha = -5 * sigmoid(a + bias)   (channel-wise, bounded to (-5, 0));
  beta      = sigmoid(b)               (one per head).
epilogue, on the core's read-out o and the output-gate projection g:
  y = RMSNorm_head(o) * w * sigmoid(g).

Readings where the pages leave a detail open (each is a parameter here):
* the short convolution is depthwise and causal with taps w[c, 0..3],
  w[c, 3] multiplying the current token and w[c, 3 - j] the token j steps
  back, no bias, zero history at a sequence start unless a cached history
  (the last three inputs before the segment) is given;
* L2 normalisation divides by sqrt(sum x^2 + eps), eps = 1e-6 by default;
* the decay bias is one value per (head, key channel);
* head RMSNorm divides by sqrt(mean o^2 + eps), eps = 1e-5 by default, with a
  weight per (head, value channel).
"""
import numpy as np

CONV_WIDTH = 4
DECAY_LOWER = -5.0


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def sigmoid(z):
    z = _f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def swish(y):
    """Swish (SiLU): y * sigmoid(y)."""
    y = _f64(y)
    return y * sigmoid(y)


def _seq_bounds(T, cu_seqlens):
    if cu_seqlens is None:
        return [(0, T)]
    cu = [int(c) for c in cu_seqlens]
    return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def short_conv(x, w, cu_seqlens=None, history=None):
    """Depthwise causal convolution of width 4 along tokens, per sequence.

    x: [T, C]; w: [C, 4]; history: [N, 3, C] (the three inputs before each
    sequence, oldest first) or None (zeros).  Returns (y [T, C], new history
    [N, 3, C]: the last three inputs of each sequence, oldest first).
    """
    x, w = _f64(x), _f64(w)
    T, C = x.shape
    bounds = _seq_bounds(T, cu_seqlens)
    y = np.zeros((T, C))
    new_hist = np.zeros((len(bounds), CONV_WIDTH - 1, C))
    for n, (bos, eos) in enumerate(bounds):
        hist = np.zeros((CONV_WIDTH - 1, C)) if history is None else _f64(history[n])
        ext = np.concatenate([hist, x[bos:eos]], axis=0)  # [3 + L, C]
        L = eos - bos
        for t in range(L):
            # ext[t + 3] is the current token, ext[t + 3 - j] the one j back
            for j in range(CONV_WIDTH):
                y[bos + t] += w[:, CONV_WIDTH - 1 - j] * ext[t + CONV_WIDTH - 1 - j]
        new_hist[n] = ext[L:L + CONV_WIDTH - 1]
    return y, new_hist


def l2_normalize(x, eps=1e-6):
    """x / sqrt(sum over the last axis of x^2 + eps)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def log_decay(a, bias):
    """Channel-wise log-decay -5 * sigmoid(a + bias), in (-5, 0).
    a: [T, H, Dk]; bias: [H, Dk]."""
    return DECAY_LOWER * sigmoid(_f64(a) + _f64(bias)[None])


def write_strength(b):
    """beta = sigmoid(b), one per (token, head)."""
    return sigmoid(b)


def head_rmsnorm(o, w, eps=1e-5):
    """o / sqrt(mean over the head's channels of o^2 + eps) * w.
    o: [T, H, Dv]; w: [H, Dv]."""
    o = _f64(o)
    r = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / r * _f64(w)[None]


def prologue(xq, xk, xv, a, b, conv_w, a_bias, cu_seqlens=None, conv_state=None,
             l2_eps=1e-6, conv=None):
    """q, k, v, log_alpha, beta (float64) and the new convolution history.

    xq, xk, xv, a: [T, H, D]; b: [T, H]; conv_w: [3, H, D, 4] (q, k, v);
    a_bias: [H, D]; conv_state: [N, 3 (q, k, v), 3 (tokens), H, D] or None.
    Returns (q, k, v, log_alpha, beta, conv_state_out [N, 3, 3, H, D]).
    `conv` (tests only) replaces the convolution step, to check that the
    pins catch a mistake in it.
    """
    conv = conv or short_conv
    xs = [_f64(xq), _f64(xk), _f64(xv)]
    T, H, D = xs[0].shape
    N = 1 if cu_seqlens is None else len(cu_seqlens) - 1
    out, states = [], np.zeros((N, 3, CONV_WIDTH - 1, H, D))
    for i, x in enumerate(xs):
        hist = None if conv_state is None else _f64(conv_state)[:, i].reshape(N, 3, H * D)
        y, nh = conv(x.reshape(T, H * D), _f64(conv_w)[i].reshape(H * D, CONV_WIDTH),
                     cu_seqlens, hist)
        states[:, i] = nh.reshape(N, 3, H, D)
        out.append(swish(y).reshape(T, H, D))
    q, k, v = out
    q, k = l2_normalize(q, l2_eps), l2_normalize(k, l2_eps)
    return q, k, v, log_decay(a, a_bias), write_strength(b), states


def epilogue(o, g, norm_w, eps=1e-5):
    """y = RMSNorm_head(o) * w * sigmoid(g); o, g: [T, H, Dv]; norm_w: [H, Dv]."""
    return head_rmsnorm(o, norm_w, eps) * sigmoid(g)
