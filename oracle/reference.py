"""Independent NumPy fp64 forms that pin the sequential oracle -- test infrastructure.

Each function is a different way of writing down what the pages describe, so a
mistake in ``kda_oracle.c`` (a dropped term, a wrong sign, a transposed operand)
shows up as a disagreement with one of them.
"""
import numpy as np


def transition(k, log_alpha, beta):
    """M_t = (I - beta k k^T) Diag(alpha), the diagonal-plus-low-rank transition of
    one token with both low-rank factors tied to the key (GeekNews "Kimi Linear"
    summary, sections "Kimi Delta Attention의 세밀한 메모리 제어" and "일반 DPLR보다
    줄어든 연산량"; a generalised Householder for alpha = 1, section "선형 어텐션에서
    Gated DeltaNet까지")."""
    k = np.asarray(k, dtype=np.float64)
    dk = k.shape[0]
    return (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(np.exp(np.asarray(log_alpha, np.float64)))


def dense_closed_form(q, k, v, log_alpha, beta, S0=None):
    """Explicit product of dense transition matrices for one sequence of one head:

        S_t = (M_t ... M_1) S_0 + sum_{s<=t} (M_t ... M_{s+1}) beta_s k_s v_s^T ,  o_t = S_t^T q_t.

    q, k, log_alpha: [T, dk]; v: [T, dv]; beta: [T]. O(T^2 d^3); tiny inputs only.
    Returns o [T, dv] and S_T [dk, dv]."""
    q, k, v, log_alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    Ms = [transition(k[t], log_alpha[t], beta[t]) for t in range(T)]

    def prod(hi, lo):  # M_hi ... M_lo (empty product = I), 0-based inclusive
        P = np.eye(dk)
        for j in range(lo, hi + 1):
            P = Ms[j] @ P
        return P

    o = np.zeros((T, dv))
    S = S0.copy()
    for t in range(T):
        S = prod(t, 0) @ S0
        for s in range(t + 1):
            S = S + prod(t, s + 1) @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = S.T @ q[t]
    return o, S


def deltanet(q, k, v, beta, S0=None):
    """Textbook delta rule (alpha = 1): read the old value with the key, blend the
    new one in with strength beta, replace. ("From GPT-2 to Kimi K3" digest, section
    "DeltaNet -- 유한한 캐시의 덮어쓰기".)

        v_old = S^T k ;  v_new = beta v + (1 - beta) v_old ;  S = S - k v_old^T + k v_new^T
    """
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        v_old = S.T @ k[t]
        v_new = beta[t] * v[t] + (1.0 - beta[t]) * v_old
        S = S - np.outer(k[t], v_old) + np.outer(k[t], v_new)
        o[t] = S.T @ q[t]
    return o, S


def gated_deltanet(q, k, v, log_gate, beta, S0=None):
    """Gated DeltaNet with one scalar decay per token ("From GPT-2 to Kimi K3"
    digest, section "Gated DeltaNet -- 망각을 더하다"), written as dense matrices:

        S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T ,  a_t = exp(log_gate_t).
    """
    q, k, v, log_gate, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_gate, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    I = np.eye(dk)
    for t in range(T):
        S = np.exp(log_gate[t]) * (I - beta[t] * np.outer(k[t], k[t])) @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def dplr_transition(a, b, log_alpha):
    """N_t = Diag(alpha_t) + a_t b_t^T, the general rank-one diagonal-plus-low-rank
    transition (GeekNews "Kimi Linear" summary, section "일반 DPLR보다 줄어든 연산량")."""
    a, b = (np.asarray(x, dtype=np.float64) for x in (a, b))
    return np.diag(np.exp(np.asarray(log_alpha, np.float64))) + np.outer(a, b)


def dplr_dense_closed_form(q, k, v, a, b, log_alpha, S0=None):
    """Explicit product of dense DPLR transitions for one sequence of one head:

        S_t = (N_t ... N_1) S_0 + sum_{s<=t} (N_t ... N_{s+1}) k_s v_s^T ,  o_t = S_t^T q_t.

    q, k, a, b, log_alpha: [T, dk]; v: [T, dv]. Tiny inputs only. Returns o, S_T."""
    q, k, v, a, b, log_alpha = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, b, log_alpha))
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    Ns = [dplr_transition(a[t], b[t], log_alpha[t]) for t in range(T)]

    def prod(hi, lo):  # N_hi ... N_lo (empty product = I), 0-based inclusive
        P = np.eye(dk)
        for j in range(lo, hi + 1):
            P = Ns[j] @ P
        return P

    o = np.zeros((T, dv))
    S = S0.copy()
    for t in range(T):
        S = prod(t, 0) @ S0
        for s in range(t + 1):
            S = S + prod(t, s + 1) @ np.outer(k[s], v[s])
        o[t] = S.T @ q[t]
    return o, S


def gated_linear_attention(q, k, v, log_alpha, S0=None):
    """Per-channel gated linear attention written as an explicit double sum (the
    DPLR recurrence with a zero low-rank term):

        o_t = sum_{s<=t} v_s sum_c q_tc k_sc e^{g_tc - g_sc} + S_0^T (q_t * e^{g_t}) ,
        g_t = sum_{j<=t} log_alpha_j.

    q, k, log_alpha: [T, dk]; v: [T, dv]. Returns o and S_T = Diag(e^{g_T}) S_0 +
    sum_s (k_s * e^{g_T - g_s}) v_s^T."""
    q, k, v, log_alpha = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha))
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    g = np.cumsum(log_alpha, axis=0)
    o = np.zeros((T, dv))
    for t in range(T):
        o[t] = S0.T @ (q[t] * np.exp(g[t]))
        for s in range(t + 1):
            o[t] += np.sum(q[t] * k[s] * np.exp(g[t] - g[s])) * v[s]
    S = np.exp(g[T - 1])[:, None] * S0 if T else S0.copy()
    for s in range(T):
        S = S + np.outer(k[s] * np.exp(g[T - 1] - g[s]), v[s])
    return o, S
