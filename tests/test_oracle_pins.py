"""Pins of the sequential fp64 oracle (CPU only).

Each test checks the C oracle against something other than itself: a hand-worked
example, exact rational arithmetic, the explicit product of dense transition
matrices, the textbook DeltaNet and Gated DeltaNet updates, exact retrieval, and
structural identities (linearity, column independence, chaining, packing, decode
steps). ``test_oracle_mutants.py`` shows that planted mistakes fail these pins.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import reference

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_case(rng, T, H, dk, dv, B=1, la_scale=0.3, normalise=True, s0=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if normalise:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    la = -la_scale * np.log1p(np.exp(rng.standard_normal((B, T, H, dk))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.3 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    f32 = lambda x: None if x is None else x.astype(np.float32)
    return tuple(map(f32, (q, k, v, la, beta))) + (None if S0 is None else S0.astype(np.float64),)


def test_hand_worked_example(oracle_lib):
    with open(os.path.join(GOLDEN, "hand_worked_d2.json")) as f:
        g = json.load(f)
    x = g["inputs"]
    q = np.array(x["q"])[None, :, None, :]
    k = np.array(x["k"])[None, :, None, :]
    v = np.array(x["v"])[None, :, None, :]
    la = np.log(np.array(x["alpha"]))[None, :, None, :]
    beta = np.array(x["beta"])[None, :, None]
    S0 = np.array(x["initial_state"])[None, None]
    o, S = oracle.forward(q, k, v, la, beta, S0)
    np.testing.assert_allclose(o[0, :, 0], np.array(g["expected"]["o"]), rtol=0, atol=1e-7)
    np.testing.assert_allclose(S[0, 0], np.array(g["expected"]["final_state"]), rtol=0, atol=1e-7)


def test_exact_rational_fixtures(oracle_lib):
    with open(os.path.join(GOLDEN, "exact_small.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        x = c["inputs"]
        fl = lambda a: np.array([[float(Fraction(s)) for s in r] for r in a])
        q, k, v = fl(x["q"]), fl(x["k"]), fl(x["v"])
        la = np.array(x["log_alpha"])
        beta = np.array([float(Fraction(s)) for s in x["beta"]])
        S0 = None if x["initial_state"] is None else fl(x["initial_state"])[None, None]
        # inputs chosen so that float32 holds them exactly, except log(alpha)
        o, S = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None], la[None, :, None],
                              beta[None, :, None], S0)
        np.testing.assert_allclose(o[0, :, 0], fl(c["expected"]["o"]), rtol=0, atol=2e-6, err_msg=c["name"])
        np.testing.assert_allclose(S[0, 0], fl(c["expected"]["final_state"]), rtol=0, atol=2e-6, err_msg=c["name"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dense_transition_product(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    T, dk, dv = 7, 5, 4
    q, k, v, la, beta, S0 = rand_case(rng, T, 1, dk, dv, la_scale=0.7)
    o, S = oracle.forward(q, k, v, la, beta, S0)
    o_ref, S_ref = reference.dense_closed_form(q[0, :, 0], k[0, :, 0], v[0, :, 0], la[0, :, 0], beta[0, :, 0], S0[0, 0])
    np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=1e-12, atol=1e-12)


def test_alpha_one_is_deltanet(oracle_lib):
    rng = np.random.default_rng(7)
    T, dk, dv = 20, 8, 6
    q, k, v, la, beta, S0 = rand_case(rng, T, 1, dk, dv)
    la = np.zeros_like(la)
    o, S = oracle.forward(q, k, v, la, beta, S0)
    o_ref, S_ref = reference.deltanet(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], S0[0, 0])
    np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=1e-12, atol=1e-12)


def test_scalar_alpha_is_gated_deltanet(oracle_lib):
    rng = np.random.default_rng(8)
    T, dk, dv = 20, 8, 6
    q, k, v, la, beta, S0 = rand_case(rng, T, 1, dk, dv)
    gate = (-0.4 * rng.random(T)).astype(np.float32)
    la = np.repeat(gate[None, :, None, None], dk, axis=-1).astype(np.float32)
    o, S = oracle.forward(q, k, v, la, beta, S0)
    o_ref, S_ref = reference.gated_deltanet(q[0, :, 0], k[0, :, 0], v[0, :, 0], gate, beta[0, :, 0], S0[0, 0])
    np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=1e-12, atol=1e-12)


def test_beta_one_unit_key_retrieves_value(oracle_lib):
    """beta = 1 and |k| = 1 overwrite what k retrieves: with q_t = k_t the output is v_t
    exactly, whatever the decay and history."""
    rng = np.random.default_rng(9)
    T, dk, dv = 40, 16, 8
    q, k, v, la, beta, S0 = rand_case(rng, T, 1, dk, dv, la_scale=2.0)
    k64 = k.astype(np.float64)
    k = (k64 / np.linalg.norm(k64, axis=-1, keepdims=True)).astype(np.float32)
    beta = np.ones_like(beta)
    o, _ = oracle.forward(k, k, v, la, beta, S0)
    kn = np.linalg.norm(k.astype(np.float64), axis=-1)
    # the float32 key is unit up to rounding; the retrieval error follows that
    tol = 1e-5 * (1 + np.abs(v).max())
    assert np.max(np.abs(kn - 1)) < 1e-6
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], rtol=0, atol=tol)


def test_orthonormal_keys_store_and_return_values(oracle_lib):
    """alpha = 1, beta = 1, orthonormal keys: every stored value is returned exactly."""
    rng = np.random.default_rng(10)
    dk, dv = 8, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T.astype(np.float32)  # rows are (nearly) orthonormal in float32
    v = rng.standard_normal((dk, dv)).astype(np.float32)
    T = dk + dk
    k_all = np.concatenate([keys, keys])[None, :, None]
    v_all = np.concatenate([v, np.zeros_like(v)])[None, :, None]
    # second pass: beta = 0 (pure reads with q = key)
    beta = np.concatenate([np.ones(dk), np.zeros(dk)]).astype(np.float32)[None, :, None]
    la = np.zeros((1, T, 1, dk), np.float32)
    o, S = oracle.forward(k_all, k_all, v_all, la, beta)
    np.testing.assert_allclose(o[0, dk:, 0], v.astype(np.float64), rtol=0, atol=1e-5)


def test_linearity(oracle_lib):
    rng = np.random.default_rng(11)
    T, H, dk, dv = 25, 2, 8, 6
    q, k, v, la, beta, S0 = rand_case(rng, T, H, dk, dv)
    _, _, v2, _, _, S02 = rand_case(rng, T, H, dk, dv)
    a, b = 0.75, -1.25
    o1, S1 = oracle.forward(q, k, v, la, beta, S0)
    o2, S2 = oracle.forward(q, k, v2, la, beta, S02)
    o3, S3 = oracle.forward(q, k, (a * v + b * v2).astype(np.float64), la, beta, a * S0 + b * S02)
    # v combination passed as float32 loses a little; compare at float32 precision
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-5)
    np.testing.assert_allclose(S3, a * S1 + b * S2, rtol=0, atol=1e-5)
    # linear in q: o(2 q) = 2 o(q) exactly (power-of-two scaling)
    o4, S4 = oracle.forward(2 * q, k, v, la, beta, S0)
    np.testing.assert_array_equal(o4, 2 * o1)
    np.testing.assert_array_equal(S4, S1)


def test_columns_and_heads_are_independent(oracle_lib):
    rng = np.random.default_rng(12)
    T, H, dk, dv = 30, 3, 8, 40
    q, k, v, la, beta, S0 = rand_case(rng, T, H, dk, dv)
    o, S = oracle.forward(q, k, v, la, beta, S0)
    o_s, S_s = oracle.forward(q, k, v, la, beta, S0, heads=[2, 0], cols=(7, 29))
    np.testing.assert_array_equal(o_s, o[:, :, [2, 0], 7:29])
    np.testing.assert_array_equal(S_s, S[:, [2, 0], :, 7:29])
    # bitwise identical for any thread count
    o1, S1 = oracle.forward(q, k, v, la, beta, S0, num_threads=1)
    np.testing.assert_array_equal(o1, o)
    np.testing.assert_array_equal(S1, S)


def test_split_and_chain(oracle_lib):
    rng = np.random.default_rng(13)
    T, H, dk, dv = 50, 2, 8, 6
    q, k, v, la, beta, S0 = rand_case(rng, T, H, dk, dv)
    o, S = oracle.forward(q, k, v, la, beta, S0)
    t = 19
    oa, Sa = oracle.forward(q[:, :t], k[:, :t], v[:, :t], la[:, :t], beta[:, :t], S0)
    ob, Sb = oracle.forward(q[:, t:], k[:, t:], v[:, t:], la[:, t:], beta[:, t:], Sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(Sb, S)


def test_varlen_equals_separate_calls(oracle_lib):
    rng = np.random.default_rng(14)
    H, dk, dv = 2, 8, 6
    lens = [5, 0, 17, 1, 9]
    T = sum(lens)
    q, k, v, la, beta, _ = rand_case(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    o, S = oracle.forward(q, k, v, la, beta, S0, cu_seqlens=cu)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        on, Sn = oracle.forward(q[:, a:b], k[:, a:b], v[:, a:b], la[:, a:b], beta[:, a:b], S0[n:n + 1])
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(S[n:n + 1], Sn)
    assert np.array_equal(S[1], S0[1])  # empty sequence: final = initial


def test_decode_steps_equal_prefill(oracle_lib):
    rng = np.random.default_rng(15)
    T, H, dk, dv = 12, 3, 8, 6
    q, k, v, la, beta, S0 = rand_case(rng, T, H, dk, dv)
    o, S = oracle.forward(q, k, v, la, beta, S0)
    state = S0.copy()
    for t in range(T):
        ot = oracle.decode_step(q[:, t], k[:, t], v[:, t], la[:, t], beta[:, t], state)
        np.testing.assert_array_equal(ot, o[:, t])
    np.testing.assert_array_equal(state, S)


def test_state_norm_bound(oracle_lib):
    """|k| = 1, alpha <= 1, beta in [0,1]: the transition has spectral norm <= 1, so
    |S_t|_2 <= |S_{t-1}|_2 + beta_t |v_t|."""
    rng = np.random.default_rng(16)
    T, dk, dv = 30, 8, 8
    q, k, v, la, beta, S0 = rand_case(rng, T, 1, dk, dv, la_scale=0.2)
    S_prev = S0[0, 0]
    state = S0.copy()
    for t in range(T):
        oracle.decode_step(q[:, t], k[:, t], v[:, t], la[:, t], beta[:, t], state)
        lhs = np.linalg.norm(state[0, 0], 2)
        rhs = np.linalg.norm(S_prev, 2) + beta[0, t, 0] * np.linalg.norm(v[0, t, 0].astype(np.float64))
        assert lhs <= rhs * (1 + 1e-6) + 1e-12
        S_prev = state[0, 0].copy()


def test_zero_length_and_zero_state(oracle_lib):
    q = np.zeros((1, 0, 1, 4), np.float32)
    o, S = oracle.forward(q, q, q, q, np.zeros((1, 0, 1), np.float32))
    assert o.shape == (1, 0, 1, 4)
    np.testing.assert_array_equal(S, 0)
