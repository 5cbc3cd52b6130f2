"""The chunkwise algebra and the in-chunk decay factoring, on the CPU in fp64,
checked against the sequential oracle. These pin the algorithm the GPU kernels
implement (the kernels share no code with either)."""
import numpy as np
import pytest

import oracle
from oracle import chunked


def one_seq(rng, T, dk, dv, la_fn):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, dv))
    la = la_fn((T, dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = 0.1 * rng.standard_normal((dk, dv))
    return [x.astype(np.float32) for x in (q, k, v, la, beta)] + [S0]


def seq_oracle(q, k, v, la, beta, S0):
    o, S = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None], la[None, :, None],
                          beta[None, :, None], S0[None, None])
    return o[0, :, 0], S[0, 0]


def test_forward_substitution_inverse():
    rng = np.random.default_rng(0)
    A = np.tril(rng.standard_normal((20, 20)) * 0.3, -1)
    T = chunked.forward_substitution_inverse(A)
    np.testing.assert_allclose(T @ (np.eye(20) + A), np.eye(20), atol=1e-12)


@pytest.mark.parametrize("C", [1, 4, 16, 64, 37])
def test_chunked_equals_sequential(oracle_lib, C):
    rng = np.random.default_rng(C)
    T, dk, dv = 37, 8, 6
    q, k, v, la, beta, S0 = one_seq(rng, T, dk, dv, lambda s: -0.2 * np.log1p(np.exp(rng.standard_normal(s))))
    o_ref, S_ref = seq_oracle(q, k, v, la, beta, S0)
    o, S = chunked.forward(q, k, v, la, beta, S0, chunk=C)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("chunk", [16, 64])
def test_factored_scheme_equals_sequential(oracle_lib, chunk):
    """The sub-chunk factoring the GPU uses (log2 units, references at sub-chunk
    boundaries) gives the sequential result; partial last chunk included."""
    rng = np.random.default_rng(21)
    T, dk, dv = 150, 16, 8
    q, k, v, la, beta, S0 = one_seq(rng, T, dk, dv, lambda s: -np.log1p(np.exp(rng.standard_normal(s))))
    o_ref, S_ref = seq_oracle(q, k, v, la, beta, S0)
    o, S = chunked.factored_forward(q, k, v, la, beta, S0, chunk=chunk)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-11)


def test_factored_fallback_branch_equals_sequential(oracle_lib):
    """Decays of -20 and -200 per token force the element-wise branch on diagonal
    sub-blocks; the result still equals the recurrence."""
    rng = np.random.default_rng(22)
    T, dk, dv = 64, 16, 8

    def la_fn(s):
        la = -0.05 * np.log1p(np.exp(rng.standard_normal(s)))
        la[5, :4] = -20.0
        la[20, 4:8] = -200.0
        la[40:45, 8:] = -30.0
        return la

    q, k, v, la, beta, S0 = one_seq(rng, T, dk, dv, la_fn)
    ops = chunked.factored_operands(q, k, la, beta, sub=16, threshold=120.0)
    assert ops["fallback"], "the adversarial decays should force the element-wise branch"
    o_ref, S_ref = seq_oracle(q, k, v, la, beta, S0)
    o, S = chunked.factored_forward(q, k, v, la, beta, S0, chunk=64)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-11)


def test_factored_operands_stay_finite_in_float32():
    """In float32 the factored operands never overflow: mixed slow/fast channels,
    and adversarial decays that take the fallback."""
    rng = np.random.default_rng(23)
    C, dk = 64, 128
    for la_case in ("mixed", "adversarial"):
        q = rng.standard_normal((C, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = rng.standard_normal((C, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        la = -np.log1p(np.exp(rng.standard_normal((C, dk))))
        if la_case == "mixed":
            la[:, rng.permutation(dk)[:64]] = -1e-3
        else:
            la[:, :32] = -20.0
            la[3, 32:64] = -200.0
        beta = 1 / (1 + np.exp(-rng.standard_normal(C)))
        with np.errstate(under="ignore"):
            ops = chunked.factored_operands(q, k, la, beta, dtype=np.float32)
            ref = chunked.factored_operands(q, k, la, beta, dtype=np.float64)
        for name in ("A", "P", "Qt", "Kt", "Kend", "gamma"):
            assert np.all(np.isfinite(ops[name])), (la_case, name)
            scale = max(1.0, np.abs(ref[name]).max())
            np.testing.assert_allclose(ops[name], ref[name], rtol=0, atol=2e-4 * scale, err_msg=f"{la_case} {name}")


def _direct_operands(q, k, la, beta):
    """A, P and the decay-scaled operands of one chunk straight from their
    definition in fp64, each pair's exponent summed over the rows it spans."""
    C = q.shape[0]
    x = la * chunked.LOG2E
    A = np.zeros((C, C))
    P = np.zeros((C, C))
    for r in range(C):
        for s in range(r + 1):
            e = np.exp2(x[s + 1:r + 1].sum(axis=0))
            P[r, s] = np.sum(q[r] * k[s] * e)
            if s < r:
                A[r, s] = beta[r] * np.sum(k[r] * k[s] * e)
    g = np.cumsum(x, axis=0)
    tail = np.stack([x[s + 1:].sum(axis=0) for s in range(C)])
    return dict(A=A, P=P, Qt=q * np.exp2(g), Kt=k * np.exp2(g), Kend=k * np.exp2(tail), gamma=np.exp2(g[-1]))


@pytest.mark.parametrize("case", ["fast12", "fast6", "two_sided", "near_limit", "mixed"])
def test_factored_operands_float32_accuracy(case):
    """In float32 the factored scheme keeps A, P and the scaled operands within 1e-5
    (normwise) of their fp64 definition, also where long runs of fast decays sit
    beside slow ones inside one sub-chunk: every exponent is a running sum of the
    decays it spans, not a difference of two long sums."""
    rng = np.random.default_rng(24)
    C, dk = 64, 128
    q = rng.standard_normal((C, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((C, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    la = -0.1 * np.log1p(np.exp(rng.standard_normal((C, dk))))
    if case == "fast12":
        la[20:32] = -200.0          # 12 tokens, every channel, then slow rows in the same sub-chunk
    elif case == "fast6":
        la[0:6] = -1000.0
    elif case == "two_sided":
        la[16] = -200.0             # fast rows at both ends of one sub-chunk
        la[31] = -200.0
    elif case == "near_limit":
        la -= 4.5                   # sub-chunk totals just inside the factoring range
    else:
        la = -np.log1p(np.exp(rng.standard_normal((C, dk))))
        la[:, rng.permutation(dk)[:64]] = -1e-3
    beta = 1 / (1 + np.exp(-rng.standard_normal(C)))
    with np.errstate(under="ignore"):
        ops = chunked.factored_operands(q, k, la, beta, dtype=np.float32)
        ref = _direct_operands(q, k, la, beta)
    assert bool(ops["fallback"]) == (case in ("fast12", "fast6", "two_sided"))
    for name in ("A", "P", "Qt", "Kt", "Kend", "gamma"):
        # values below float32's smallest normal number are out of its range: zero
        want = np.where(np.abs(ref[name]) < np.finfo(np.float32).tiny, 0.0, ref[name])
        nref = np.linalg.norm(want)
        err = np.linalg.norm(np.where(np.abs(want) > 0, ops[name], 0.0) - want) / (nref if nref > 0 else 1.0)
        assert err <= 1e-5, (case, name, err)
        assert np.all(np.abs(ops[name][want == 0]) <= np.finfo(np.float32).tiny), (case, name)
