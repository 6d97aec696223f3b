"""Brute-force evaluation of the KDA equation with explicit matrices.

Test infrastructure: an evaluation of the published equation that is
independent of the oracle's order of operations.  Each token's transition is
built as the explicit d_k x d_k matrix

    M_t = (I - beta_t k_t k_t^T) Diag(alpha_t)

("Kimi K3 Architecture Explained", Step 3, the KDA equation; "An
infra-oriented diagram of Kimi K3", KDA card) and the final state is the
unrolled sum

    S_T = M_T ... M_1 S_0 + sum_s M_T ... M_{s+1} beta_s k_s v_s^T,

with o_t = S_t^T q_t taken from the partial sums.  Only for tiny T (the
products are O(T^2 d^3)).
"""
import numpy as np


def transition(k, log_alpha, beta):
    """M = (I - beta k k^T) Diag(exp(log_alpha)) as an explicit matrix."""
    d = k.shape[0]
    return (np.eye(d) - beta * np.outer(k, k)) @ np.diag(np.exp(log_alpha))


def unrolled(q, k, v, log_alpha, beta, S0):
    """q, k, log_alpha: [T, Dk]; v: [T, Dv]; beta: [T]; S0: [Dk, Dv].

    Returns (o [T, Dv], S_T) evaluated as sums of products of transition
    matrices (no running state is updated in place)."""
    T = q.shape[0]
    M = [transition(k[t], log_alpha[t], beta[t]) for t in range(T)]
    W = [beta[t] * np.outer(k[t], v[t]) for t in range(T)]
    o = np.zeros((T, v.shape[1]))
    S_t = None
    for t in range(T):
        # S_t = (M_t ... M_1) S0 + sum_{s<=t} (M_t ... M_{s+1}) W_s
        P = np.eye(k.shape[1])
        acc = np.zeros_like(S0, dtype=np.float64)
        for s in range(t, -1, -1):
            acc = acc + P @ W[s]
            P = P @ M[s]
        S_t = P @ S0 + acc
        o[t] = S_t.T @ q[t]
    return o, (S0.copy() if S_t is None else S_t)


def affine_segment(k, log_alpha, beta, v):
    """The segment's affine map S -> A S + B as explicit matrices
    (A = M_T ... M_1, B = the zero-state result)."""
    d = k.shape[1]
    A = np.eye(d)
    B = np.zeros((d, v.shape[1]))
    for t in range(k.shape[0]):
        Mt = transition(k[t], log_alpha[t], beta[t])
        A = Mt @ A
        B = Mt @ B + beta[t] * np.outer(k[t], v[t])
    return A, B
