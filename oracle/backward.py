"""CPU oracle for the KDA backward pass -- TEST INFRASTRUCTURE ONLY (same
rule as the rest of ``oracle``).

The pages give the forward recurrence only ("Kimi K3 Architecture
Explained", Step 3; the KDA card of "An infra-oriented diagram of Kimi K3";
training runs the chunkwise mode, "From GPT-2 to Kimi K3", ch. 6).  The
gradients here are reverse-mode differentiation of that token-by-token
recurrence, one step at a time, in float64, written as the four steps of
a token in reverse:

  forward, per token t and head:
    S'  = Diag(alpha_t) S_{t-1},            alpha_t = exp(log_alpha_t)
    p   = S'^T k_t
    u   = beta_t (v_t - p)
    S_t = S' + k_t u^T
    o_t = S_t^T q_t
  reverse, with dS = dLoss/dS_t accumulated from later tokens:
    dS += q_t do_t^T;            dq_t = S_t do_t
    du  = dS^T k_t;              dk_t = dS u
    dbeta_t = du . (v_t - p);    dv_t = beta_t du;    dp = -beta_t du
    dS' = dS + k_t dp^T;         dk_t += S' dp
    dlog_alpha_t = alpha_t o sum_j (dS' o S_{t-1})[:, j]
    dS  = Diag(alpha_t) dS'      (the gradient of S_{t-1})
  and dh0 = dS after the first token of each sequence.

The loss is sum(do * o) + sum(dh_T * h_T), so (do, dh_T) are the incoming
gradients.  Pinned in tests/test_oracle_backward_pins.py by finite
differences of the C forward oracle (a separate implementation), closed
forms and special cases.
"""
import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _bounds(T, cu_seqlens):
    if cu_seqlens is None:
        return [(0, T)]
    cu = [int(c) for c in cu_seqlens]
    return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def bwd(q, k, v, log_alpha, beta, do, dhT=None, h0=None, cu_seqlens=None):
    """Gradients of sum(do * o) + sum(dhT * h_T) for the KDA forward pass.

    q, k, log_alpha: [T, H, Dk]; v, do: [T, H, Dv]; beta: [T, H];
    h0, dhT: [N, H, Dk, Dv] or None (zero).  Returns (dq, dk, dv,
    dlog_alpha, dbeta, dh0) in float64, shaped like the inputs (dh0
    [N, H, Dk, Dv]).
    """
    q, k, v, g, b, do = (_f64(x) for x in (q, k, v, log_alpha, beta, do))
    T, H, Dk = q.shape
    Dv = v.shape[2]
    bounds = _bounds(T, cu_seqlens)
    N = len(bounds)
    h0, dhT = _f64(h0), _f64(dhT)
    dq, dk, dv, dg = (np.zeros_like(x) for x in (q, k, v, g))
    db = np.zeros_like(b)
    dh0 = np.zeros((N, H, Dk, Dv))
    for n, (bos, eos) in enumerate(bounds):
        L = eos - bos
        for h in range(H):
            # forward, keeping every state (S[0] = h0, S[t + 1] after token t)
            S = np.zeros((L + 1, Dk, Dv))
            if h0 is not None:
                S[0] = h0[n, h]
            Sp = np.zeros((L, Dk, Dv))
            P = np.zeros((L, Dv))
            Uu = np.zeros((L, Dv))
            for t in range(L):
                r = bos + t
                a = np.exp(g[r, h])
                Sp[t] = a[:, None] * S[t]
                P[t] = Sp[t].T @ k[r, h]
                Uu[t] = b[r, h] * (v[r, h] - P[t])
                S[t + 1] = Sp[t] + np.outer(k[r, h], Uu[t])
            # reverse
            dS = np.zeros((Dk, Dv)) if dhT is None else dhT[n, h].copy()
            for t in range(L - 1, -1, -1):
                r = bos + t
                a = np.exp(g[r, h])
                dS += np.outer(q[r, h], do[r, h])
                dq[r, h] = S[t + 1] @ do[r, h]
                du = dS.T @ k[r, h]
                dk[r, h] = dS @ Uu[t]
                db[r, h] = du @ (v[r, h] - P[t])
                dv[r, h] = b[r, h] * du
                dp = -b[r, h] * du
                dSp = dS + np.outer(k[r, h], dp)
                dk[r, h] += Sp[t] @ dp
                dg[r, h] = a * np.sum(dSp * S[t], axis=1)
                dS = a[:, None] * dSp
            dh0[n, h] = dS
    return dq, dk, dv, dg, db, dh0
