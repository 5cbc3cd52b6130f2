"""Exact rational evaluation of the KDA recurrence for tiny inputs -- test infrastructure.

Uses ``fractions.Fraction`` so that there is no rounding at all. The decay is
given directly as a rational alpha in (0, 1] (the floating-point paths receive
log(alpha)). The state is propagated with explicit dense transition matrices

    S_t = M_t S_{t-1} + beta_t k_t v_t^T ,   M_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
    o_t = S_t^T q_t ,

the diagonal-plus-low-rank transition of the GeekNews "Kimi Linear" summary,
section "Kimi Delta Attention의 세밀한 메모리 제어".
"""
from fractions import Fraction


def _mat(rows, cols, val=Fraction(0)):
    return [[val for _ in range(cols)] for _ in range(rows)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)] for i in range(n)]


def forward_exact(q, k, v, alpha, beta, S0=None):
    """q, k, alpha: T lists of dk Fractions; v: T lists of dv Fractions; beta: T Fractions.
    Returns (o, S_T) as nested lists of Fractions."""
    T = len(q)
    dk = len(k[0])
    dv = len(v[0])
    S = _mat(dk, dv) if S0 is None else [list(map(Fraction, row)) for row in S0]
    outs = []
    for t in range(T):
        M = _mat(dk, dk)
        for i in range(dk):
            for j in range(dk):
                M[i][j] = ((Fraction(1) if i == j else Fraction(0)) - beta[t] * k[t][i] * k[t][j]) * alpha[t][j]
        S = _matmul(M, S)
        for i in range(dk):
            for j in range(dv):
                S[i][j] += beta[t] * k[t][i] * v[t][j]
        outs.append([sum((S[i][j] * q[t][i] for i in range(dk)), Fraction(0)) for j in range(dv)])
    return outs, S
