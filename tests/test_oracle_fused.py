"""Pins for the oracle's prologue and epilogue (oracle/fused.py and the C prologue).

The activations are pinned by identities and closed forms that do not reuse their
own formulas; the C prologue is pinned against the explicit dense-product form fed
with inputs transformed in NumPy."""
import numpy as np
import pytest

import oracle
from oracle import fused, reference, seq


def test_softplus_identities():
    x = np.concatenate([np.linspace(-40, 40, 161), [-700.0, -50.0, 0.0, 50.0, 700.0]])
    sp = fused.softplus(x)
    assert np.all(np.isfinite(sp))
    # softplus(x) - softplus(-x) = x, softplus(x) >= max(x, 0)
    np.testing.assert_allclose(sp - fused.softplus(-x), x, rtol=0, atol=1e-12)
    assert np.all(sp >= np.maximum(x, 0.0))
    assert fused.softplus(0.0) == pytest.approx(np.log(2.0), abs=1e-15)
    # tails: softplus(x) -> x and softplus(-x) -> e^-x
    assert fused.softplus(40.0) - 40.0 == pytest.approx(np.exp(-40.0), rel=1e-6)
    assert fused.softplus(-40.0) == pytest.approx(np.exp(-40.0), rel=1e-12)


def test_sigmoid_identities_and_derivative():
    x = np.linspace(-30, 30, 121)
    s = fused.sigmoid(x)
    np.testing.assert_allclose(s + fused.sigmoid(-x), 1.0, atol=1e-15)
    np.testing.assert_allclose(s, np.exp(x) / (1.0 + np.exp(x)), rtol=1e-13)
    assert fused.sigmoid(0.0) == 0.5
    # d softplus / dx = sigmoid, by central differences
    h = 1e-5
    np.testing.assert_allclose((fused.softplus(x + h) - fused.softplus(x - h)) / (2 * h), s, atol=1e-9)
    assert np.all(np.isfinite(fused.sigmoid(np.array([-800.0, 800.0]))))


def test_gate_is_sigmoid_of_negated_preactivation():
    # alpha = exp(-softplus(a)) = 1 / (1 + e^a)
    a = np.linspace(-20, 20, 81)
    np.testing.assert_allclose(np.exp(fused.gate_log_alpha(a)), 1.0 / (1.0 + np.exp(a)), rtol=1e-12)
    assert np.all(fused.gate_log_alpha(a) < 0)


def test_l2_normalize():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 128)) * rng.uniform(0.1, 10.0, (7, 1))
    y = fused.l2_normalize(x, 1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-9)
    np.testing.assert_allclose(fused.l2_normalize(3.7 * x, 0.0), fused.l2_normalize(x, 0.0), atol=1e-15)
    # same direction: y = x / ||x||
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-9)
    assert np.all(fused.l2_normalize(np.zeros((2, 128)), 1e-6) == 0.0)


def test_output_norm_gate_closed_forms():
    w = np.linspace(0.5, 1.5, 128)
    for c in (-3.0, 0.25, 2.0):
        o = np.full((1, 128), c)
        y = fused.output_norm_gate(o, np.zeros((1, 128)), w, 1e-6)
        np.testing.assert_allclose(y[0], np.sign(c) * abs(c) / np.sqrt(c * c + 1e-6) * w * 0.5, rtol=1e-14)
    rng = np.random.default_rng(1)
    o = rng.standard_normal((5, 128))
    z = rng.standard_normal((5, 128))
    y = fused.output_norm_gate(o, z, np.ones(128), 0.0)
    g = 1.0 / (1.0 + np.exp(-z))
    np.testing.assert_allclose(np.sqrt(np.mean((y / g) ** 2, axis=-1)), 1.0, atol=1e-12)
    np.testing.assert_allclose(fused.output_norm_gate(5.0 * o, z, np.ones(128), 0.0), y, atol=1e-13)


def _raw(rng, T, dk, dv):
    q = rng.standard_normal((T, dk)) * 2.0
    k = rng.standard_normal((T, dk)) * 0.5
    v = rng.standard_normal((T, dv))
    a = rng.standard_normal((T, dk))
    b = rng.standard_normal(T)
    return [np.asarray(x, np.float32) for x in (q, k, v, a, b)]


@pytest.mark.parametrize("eps", [0.0, 1e-3])
def test_c_prologue_matches_dense_form(eps):
    rng = np.random.default_rng(2)
    T, dk, dv = 7, 5, 4
    q, k, v, a, b = _raw(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv)) * 0.1
    # the prologue in NumPy, written with different formulas
    qn = q.astype(np.float64) / np.sqrt((q.astype(np.float64) ** 2).sum(-1, keepdims=True) + eps)
    kn = k.astype(np.float64) / np.sqrt((k.astype(np.float64) ** 2).sum(-1, keepdims=True) + eps)
    la = -np.log1p(np.exp(a.astype(np.float64)))
    beta = 1.0 / (1.0 + np.exp(-b.astype(np.float64)))
    o_ref, S_ref = reference.dense_closed_form(qn, kn, v, la, beta, S0)
    flags = seq.prologue_flags(True, True, True)
    o, S = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None], a[None, :, None],
                          b[None, :, None], S0[None, None], flags=flags, qk_eps=eps)
    np.testing.assert_allclose(o[0, :, 0], o_ref, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], S_ref, atol=1e-12)
    # the decode step applies the same prologue
    st = S0[None, None].copy()
    od = oracle.decode_step(q[None, :1], k[None, :1], v[None, :1], a[None, :1], b[None, :1], st,
                            flags=flags, qk_eps=eps)
    o1, S1 = reference.dense_closed_form(qn[:1], kn[:1], v[:1], la[:1], beta[:1], S0)
    np.testing.assert_allclose(od[0, 0], o1[0], atol=1e-12)
    np.testing.assert_allclose(st[0, 0], S1, atol=1e-12)


def test_each_prologue_flag_acts_alone():
    """Each flag changes exactly its own input: with the others off, the result
    equals the plain oracle fed that one input transformed in NumPy."""
    rng = np.random.default_rng(3)
    T, dk, dv = 9, 6, 3
    q, k, v, a, b = _raw(rng, T, dk, dv)
    la = (-np.abs(a) * 0.3).astype(np.float32)
    bb = (1.0 / (1.0 + np.exp(-b))).astype(np.float32)
    args = lambda *xs: [x[None, :, None] for x in xs]  # noqa: E731
    # gate only: feed softplus^{-1}(-la) as the pre-activation
    pre = np.log(np.expm1(-la.astype(np.float64))).astype(np.float32)
    o1, _ = oracle.forward(*args(q, k, v, pre, bb), flags=seq.GATE_PRE)
    o0, _ = oracle.forward(*args(q, k, v, np.float32(-np.log1p(np.exp(pre.astype(np.float64)))), bb))
    np.testing.assert_allclose(o1, o0, atol=1e-6)
    # beta only
    o1, _ = oracle.forward(*args(q, k, v, la, b), flags=seq.BETA_PRE)
    o0, _ = oracle.forward(*args(q, k, v, la, (1.0 / (1.0 + np.exp(-b.astype(np.float64)))).astype(np.float32)))
    np.testing.assert_allclose(o1, o0, atol=1e-6)
    # normalisation only: unit-norm inputs are (nearly) unchanged by it
    qu = (q / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32)
    ku = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    o1, _ = oracle.forward(*args(q, k, v, la, bb), flags=seq.NORM_QK)
    o0, _ = oracle.forward(*args(qu, ku, v, la, bb))
    np.testing.assert_allclose(o1, o0, atol=1e-6)


def test_fused_forward_applies_epilogue_per_row():
    rng = np.random.default_rng(4)
    B, T, H, d = 1, 10, 3, 8
    q, k, v, a = (rng.standard_normal((B, T, H, d)).astype(np.float32) for _ in range(4))
    b = rng.standard_normal((B, T, H)).astype(np.float32)
    z = rng.standard_normal((B, T, H, d)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, d)
    o_plain, _ = fused.forward(q, k, v, a, b)
    o, _ = fused.forward(q, k, v, a, b, out_gate=z, norm_weight=w, norm_eps=1e-5)
    for h in range(H):
        for t in range(T):
            row = o_plain[0, t, h]
            expect = row / np.sqrt(np.mean(row ** 2) + 1e-5) * w / (1.0 + np.exp(-z[0, t, h].astype(np.float64)))
            np.testing.assert_allclose(o[0, t, h], expect, rtol=1e-12)
    # a head subset gives the same rows
    o2, _ = fused.forward(q, k, v, a, b, out_gate=z, norm_weight=w, norm_eps=1e-5, heads=[2, 0])
    np.testing.assert_allclose(o2[:, :, 0], o[:, :, 2], rtol=1e-13)
    np.testing.assert_allclose(o2[:, :, 1], o[:, :, 0], rtol=1e-13)
