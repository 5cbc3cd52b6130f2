"""Chunkwise (WY / UT transform) form of the KDA recurrence -- test infrastructure.

These functions pin the algebra the GPU kernels implement against the
sequential oracle on the CPU. They share no code with the GPU library.

Chunking follows "From GPT-2 to Kimi K3" digest, section "DeltaNet 병렬화 --
청크 단위 학습" (split T into chunks of C; in-chunk work is masked attention, the
rest is carried by the state), and the GeekNews "Kimi Linear" summary, section
"청크 단위 병렬 알고리듬": a WY representation packs the chunk's rank-one updates,
the UT transform applies (I + A)^{-1}, and the lower-triangular inverse is found
row by row by forward substitution.

Per chunk (rows r, s; g_r = sum_{j<=r} log_alpha_j per channel; S_0 the state
entering the chunk):
    A_rs = beta_r sum_c k_rc k_sc e^{g_rc - g_sc}              (s < r)
    T    = (I + A)^{-1}
    W    = T diag(beta) (K * e^G) ,  U = T diag(beta) V
    U~   = U - W S_0
    P_rs = sum_c q_rc k_sc e^{g_rc - g_sc}                      (s <= r)
    O    = (Q * e^G) S_0 + P U~
    S_C  = Diag(e^{g_C}) S_0 + (K * e^{g_C - G})^T U~
Derivation: write S_t = Diag(alpha_t) S_{t-1} + k_t u_t^T with
u_t = beta_t (v_t - (Diag(alpha_t) S_{t-1})^T k_t); unrolling inside the chunk gives
(I + A) U~ = diag(beta) (V - (K * e^G) S_0).
"""
import numpy as np

LOG2E = 1.4426950408889634


def forward_substitution_inverse(A):
    """T = (I + A)^{-1} for strictly lower-triangular A, one row at a time:
    T_r = e_r - sum_{s<r} A_rs T_s (Gaussian elimination, forward substitution)."""
    C = A.shape[0]
    T = np.zeros_like(A)
    for r in range(C):
        row = np.zeros(C, dtype=A.dtype)
        row[r] = 1.0
        for s in range(r):
            row = row - A[r, s] * T[s]
        T[r] = row
    return T


def chunk_step(q, k, v, log_alpha, beta, S0):
    """One chunk of the plain chunked form in fp64 with e^{+-G} taken directly.
    q, k, log_alpha: [C, dk]; v: [C, dv]; beta: [C]; S0: [dk, dv]."""
    g = np.cumsum(log_alpha, axis=0)
    C = q.shape[0]
    Kp, Km = k * np.exp(g), k * np.exp(-g)
    A = np.tril(beta[:, None] * (Kp @ Km.T), -1)
    T = forward_substitution_inverse(A)
    W = T @ (beta[:, None] * Kp)
    U = T @ (beta[:, None] * v)
    Ut = U - W @ S0
    P = np.tril((q * np.exp(g)) @ Km.T)
    O = (q * np.exp(g)) @ S0 + P @ Ut
    gC = g[C - 1]
    S = np.exp(gC)[:, None] * S0 + (k * np.exp(gC[None, :] - g)).T @ Ut
    return O, S


def forward(q, k, v, log_alpha, beta, S0=None, chunk=64, step=chunk_step):
    """Chunked fp64 KDA for one sequence of one head. The last chunk may be
    partial. q, k, log_alpha: [T, dk]; v: [T, dv]; beta: [T]."""
    q, k, v, log_alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        o[t0:t1], S = step(q[t0:t1], k[t0:t1], v[t0:t1], log_alpha[t0:t1], beta[t0:t1], S)
    return o, S


# ---------------------------------------------------------------------------
# In-chunk decay factoring with a fallback, emulated on the CPU.
#
# e^{g_r - g_s} with g_r - g_s <= 0 is always safe, but the matmul form splits it
# into e^{g_r} * e^{-g_s}, which overflows for fast decays (the GeekNews summary,
# section "일반 DPLR보다 줄어든 연산량", notes that fine-grained decay makes in-chunk
# division numerically delicate; GLA handles it with log-space, full-precision
# secondary chunking). The scheme here works in log2 units (x = log2 alpha), splits
# the chunk into sub-chunks of `sub` rows, and keeps every exponent a sum of the
# decays it spans, never the difference of two long sums, so rounding stays
# relative to the exponent itself:
#   loc_r = x over rows [start of r's sub-chunk, r]        (running sum, <= 0)
#   suf_s = x over rows (s, end of s's sub-chunk]          (reverse running sum, <= 0)
#   R_I   = x over sub-chunk I (= loc at its last row);  b_I = R_0 + ... + R_{I-1}
#   pair r >= s, r in sub-chunk I, s in sub-chunk J:
#     gh_r - gh_s = loc_r + E_IJ + suf_s,   E_IJ = R_{J+1} + ... + R_{I-1} (J < I),
#                                           E_II = -R_I
#   the operands: plus_r = 2^(loc_r), minus_s = 2^(suf_s), both in (0, 1]; the block
#   scale 2^(E_IJ) is <= 1 off the diagonal and 2^(-R_I) on it.
#   When -R_I > threshold for some sub-chunk its diagonal block is formed element by
#   element with 2^(gh_r - gh_s) (exponent <= 0), the exponent taken as
#   loc_r - loc_s or suf_s - suf_r, whichever subtracts the smaller sum (the decay
#   before s or after r inside the sub-chunk).
#   Q~ = q * 2^(b_I + loc);  K~ = k * 2^(b_I + loc);
#   K~end_s = k_s * minus_s * 2^(R_{J+1} + ... + R_{n-1});  gamma = 2^(b_n).
# ---------------------------------------------------------------------------

def _local_sums(x, sub, dtype):
    """Running sums of x inside each sub-chunk, forward (loc) and backward (suf),
    and the sub-chunk totals R, all accumulated row by row in ``dtype``."""
    C, dk = x.shape
    n_sub = (C + sub - 1) // sub
    loc = np.zeros((C, dk), dtype=dtype)
    suf = np.zeros((C, dk), dtype=dtype)
    R = np.zeros((n_sub, dk), dtype=dtype)
    for I in range(n_sub):
        rows = range(sub * I, min(C, sub * (I + 1)))
        acc = np.zeros(dk, dtype=dtype)
        for r in rows:
            acc = (acc + x[r]).astype(dtype)
            loc[r] = acc
        R[I] = acc
        acc = np.zeros(dk, dtype=dtype)
        for s in reversed(rows):
            suf[s] = acc
            acc = (acc + x[s]).astype(dtype)
    return loc, suf, R


def _span(R, lo, hi, dtype):
    """R_lo + ... + R_{hi-1} (zero when empty), accumulated in ``dtype``."""
    acc = np.zeros(R.shape[1], dtype=dtype)
    for K in range(lo, hi):
        acc = (acc + R[K]).astype(dtype)
    return acc


def factored_operands(q, k, log_alpha, beta, sub=16, threshold=120.0, dtype=np.float64):
    """Forms A, P, Q~, K~, K~end, gamma of one chunk with the factored scheme, in
    ``dtype`` arithmetic. Returns a dict with those and ``fallback`` (list of the
    diagonal sub-blocks that took the element-wise path)."""
    C, dk = q.shape
    n_sub = (C + sub - 1) // sub
    x = (np.asarray(log_alpha, dtype=np.float64) * LOG2E).astype(dtype)
    loc, suf, R = _local_sums(x, sub, dtype)
    b = np.zeros((n_sub + 1, dk), dtype=dtype)
    for I in range(n_sub):
        b[I + 1] = (b[I] + R[I]).astype(dtype)
    q = np.asarray(q, dtype=dtype)
    k = np.asarray(k, dtype=dtype)
    beta = np.asarray(beta, dtype=dtype)
    plus = np.exp2(loc)
    minus = np.exp2(suf)
    A = np.zeros((C, C), dtype=dtype)
    P = np.zeros((C, C), dtype=dtype)
    fallback = []
    over = [I for I in range(n_sub) if np.max(-R[I]) > threshold]
    with np.errstate(over="raise", invalid="raise"):
        for I in range(n_sub):
            rI = slice(sub * I, min(C, sub * (I + 1)))
            lhs_k = k[rI] * plus[rI]
            lhs_q = q[rI] * plus[rI]
            for J in range(I + 1):
                sJ = slice(sub * J, min(C, sub * (J + 1)))
                if J < I or I not in over:
                    scale = np.exp2(_span(R, J + 1, I, dtype) if J < I else -R[I])
                    rhs = k[sJ] * minus[sJ] * scale
                    blkA = lhs_k @ rhs.T
                    blkP = lhs_q @ rhs.T
                else:
                    fallback.append(I)
                    rows = range(rI.start, rI.stop)
                    blkA = np.zeros((len(rows), len(rows)), dtype=dtype)
                    blkP = np.zeros_like(blkA)
                    for a, r in enumerate(rows):
                        for c, s in enumerate(rows):
                            if s <= r:
                                near = np.abs(loc[s]) <= np.abs(suf[r])
                                e = np.exp2(np.where(near, loc[r] - loc[s], suf[s] - suf[r]))
                                blkA[a, c] = np.sum(k[r] * k[s] * e)
                                blkP[a, c] = np.sum(q[r] * k[s] * e)
                if J == I:
                    n = blkA.shape[0]
                    blkA = np.where(np.tril(np.ones((n, n), bool), -1), blkA, 0)
                    blkP = np.where(np.tril(np.ones((n, n), bool), 0), blkP, 0)
                A[rI, sJ] = blkA
                P[rI, sJ] = blkP
        A = beta[:, None] * A
        blk_of = np.arange(C) // sub
        eg = np.exp2(b[blk_of] + loc)
        Qt = q * eg
        Kt = k * eg
        tail = np.stack([_span(R, J + 1, n_sub, dtype) for J in range(n_sub)])
        Kend = k * minus * np.exp2(tail[blk_of])
        gamma = np.exp2(b[n_sub])
    return dict(A=A, P=P, Qt=Qt, Kt=Kt, Kend=Kend, gamma=gamma, fallback=fallback)


def factored_chunk_step(q, k, v, log_alpha, beta, S0, sub=16, threshold=120.0):
    """A chunk step in which every decay factor comes from the factored scheme."""
    op = factored_operands(q, k, log_alpha, beta, sub=sub, threshold=threshold)
    T = forward_substitution_inverse(op["A"])
    W = T @ (beta[:, None] * op["Kt"])
    U = T @ (beta[:, None] * v)
    Ut = U - W @ S0
    O = op["Qt"] @ S0 + op["P"] @ Ut
    S = op["gamma"][:, None] * S0 + op["Kend"].T @ Ut
    return O, S


def factored_forward(q, k, v, log_alpha, beta, S0=None, chunk=64, sub=16, threshold=120.0):
    return forward(q, k, v, log_alpha, beta, S0, chunk,
                   step=lambda *a: factored_chunk_step(*a, sub=sub, threshold=threshold))


# ---------------------------------------------------------------------------
# Chunkwise form of the general DPLR recurrence
#     S_t = (Diag(alpha_t) + a_t b_t^T) S_{t-1} + k_t v_t^T ,  o_t = S_t^T q_t
# (GeekNews "Kimi Linear" summary, section "일반 DPLR보다 줄어든 연산량": a general
# DPLR transition needs four secondary C x C matrices per chunk where KDA needs two).
# With w_t = S_{t-1}^T b_t the state is S_t = Diag(alpha_t) S_{t-1} + a_t w_t^T +
# k_t v_t^T. Per chunk (g inclusive and g^- = g - log_alpha exclusive cumulative
# log-decays, S_0 the state entering the chunk):
#   M_ba[r,s] = sum_c b_rc a_sc e^{g^-_rc - g_sc}   (s < r)     M_bk: k_s in place of a_s
#   M_qa[r,s] = sum_c q_rc a_sc e^{g_rc - g_sc}     (s <= r)    M_qk: k_s in place of a_s
#   T   = (I - M_ba)^{-1}
#   W   = T (B * e^{G^-}) S_0 + T M_bk V                        (rows w_r)
#   O   = (Q * e^G) S_0 + M_qa W + M_qk V
#   S_C = Diag(e^{g_C}) S_0 + (A * e^{g_C - G})^T W + (K * e^{g_C - G})^T V
# Derivation: unrolling inside the chunk, w_r = S_0^T (b_r e^{g^-_r}) + sum_{s<r}
# [M_ba]_rs w_s + [M_bk]_rs v_s, i.e. (I - M_ba) W = (B e^{G^-}) S_0 + M_bk V; the
# output and the chunk-end state follow by substituting S_r.
# ---------------------------------------------------------------------------
def dplr_chunk_step(q, k, v, a, b, log_alpha, S0):
    """One chunk of the DPLR chunked form in fp64, exponentials taken directly."""
    g = np.cumsum(log_alpha, axis=0)
    gm = g - log_alpha
    C = q.shape[0]
    lower = np.tril(np.ones((C, C)), -1)
    incl = np.tril(np.ones((C, C)))
    d_ex = np.exp(gm[:, None, :] - g[None, :, :])   # [r, s, c] e^{g^-_r - g_s}
    d_in = np.exp(g[:, None, :] - g[None, :, :])    # [r, s, c] e^{g_r - g_s}
    M_ba = lower * np.einsum("rc,sc,rsc->rs", b, a, d_ex * lower[:, :, None])
    M_bk = lower * np.einsum("rc,sc,rsc->rs", b, k, d_ex * lower[:, :, None])
    M_qa = incl * np.einsum("rc,sc,rsc->rs", q, a, d_in * incl[:, :, None])
    M_qk = incl * np.einsum("rc,sc,rsc->rs", q, k, d_in * incl[:, :, None])
    T = np.linalg.inv(np.eye(C) - M_ba)
    W = T @ (b * np.exp(gm)) @ S0 + T @ M_bk @ v
    O = (q * np.exp(g)) @ S0 + M_qa @ W + M_qk @ v
    gC = g[C - 1]
    S = np.exp(gC)[:, None] * S0 + (a * np.exp(gC[None, :] - g)).T @ W + (k * np.exp(gC[None, :] - g)).T @ v
    return O, S


def dplr_forward(q, k, v, a, b, log_alpha, S0=None, chunk=64):
    """Chunked fp64 DPLR for one sequence of one head (the last chunk may be partial).
    q, k, a, b, log_alpha: [T, dk]; v: [T, dv]."""
    q, k, v, a, b, log_alpha = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, b, log_alpha))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        o[t0:t1], S = dplr_chunk_step(q[t0:t1], k[t0:t1], v[t0:t1], a[t0:t1], b[t0:t1], log_alpha[t0:t1], S)
    return o, S
