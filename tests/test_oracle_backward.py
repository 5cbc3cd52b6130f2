"""Pins of the oracle's backward (``kda_oracle_backward``), CPU only.

The gradients are pinned against things other than the oracle itself:
  - central finite differences of the explicit dense-matrix forward
    (``reference.dense_closed_form``, written independently of the C recurrence),
    one input tensor at a time, with varlen sequences, a non-zero initial state and
    a cotangent on the final state;
  - reverse mode by torch.autograd through an independently written fp64 torch
    recurrence (dense transition matrices), over sequences longer than the C
    oracle's checkpoint segment;
  - the chain rule across a split sequence (state passing), and linearity in the
    cotangents.
Planted mistakes in copies of the backward must fail the finite-difference pin.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import reference

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "kda_oracle.c")


def _inputs(rng, B, T, H, dk, dv, decay=0.4):
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    q = rng.standard_normal((B, T, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    la = -decay * rng.random((B, T, H, dk))
    beta = rng.random((B, T, H))
    return tuple(map(f32, (q, k, v, la, beta)))


def _loss_dense(q, k, v, la, beta, S0, do, dfin, starts):
    """L = sum <o, do> + sum <S_final, dfin> with the dense-matrix forward, fp64."""
    H = q.shape[2]
    L = 0.0
    for n in range(len(starts) - 1):
        a, b = starts[n], starts[n + 1]
        for h in range(H):
            o, S = reference.dense_closed_form(q[0, a:b, h], k[0, a:b, h], v[0, a:b, h], la[0, a:b, h],
                                               beta[0, a:b, h], S0[n, h])
            L += float(np.sum(o * do[0, a:b, h])) + float(np.sum(S * dfin[n, h]))
    return L


def _fd_case(seed=3):
    rng = np.random.default_rng(seed)
    dk, dv, H = 6, 5, 2
    starts = np.array([0, 3, 8])
    T = int(starts[-1])
    q, k, v, la, beta = _inputs(rng, 1, T, H, dk, dv)
    S0 = rng.standard_normal((2, H, dk, dv))
    do = rng.standard_normal((1, T, H, dv)).astype(np.float32)
    dfin = rng.standard_normal((2, H, dk, dv))
    return dict(q=q, k=k, v=v, la=la, beta=beta, S0=S0, do=do, dfin=dfin, starts=starts)


def fd_failures(lib=None, seed=3, eps=1e-5, rtol=1e-6):
    """Names of the gradients whose directional derivative disagrees with central
    finite differences of the dense forward."""
    c = _fd_case(seed)
    g = oracle.backward(c["q"], c["k"], c["v"], c["la"], c["beta"], d_o=c["do"], initial_state=c["S0"],
                        d_final=c["dfin"], cu_seqlens=c["starts"], lib=lib)
    rng = np.random.default_rng(seed + 100)
    base = {n: np.asarray(c[n], dtype=np.float64) for n in ("q", "k", "v", "la", "beta", "S0")}
    grads = {"q": g["dq"], "k": g["dk"], "v": g["dv"], "la": g["dlog_alpha"], "beta": g["dbeta"],
             "S0": g["d_initial"]}
    failed = []
    for name in base:
        U = rng.standard_normal(base[name].shape)
        args_p = dict(base); args_p[name] = base[name] + eps * U
        args_m = dict(base); args_m[name] = base[name] - eps * U
        call = lambda a: _loss_dense(a["q"], a["k"], a["v"], a["la"], a["beta"], a["S0"], c["do"], c["dfin"],
                                     c["starts"])
        fd = (call(args_p) - call(args_m)) / (2 * eps)
        an = float(np.sum(grads[name] * U))
        if not abs(fd - an) <= rtol * (abs(fd) + 1.0):
            failed.append(name)
    return failed


def test_gradients_match_finite_differences_of_the_dense_form():
    assert fd_failures() == []


def _torch_recurrence(q, k, v, la, beta, S0, starts):
    """fp64 torch recurrence with dense transitions M_t = (I - beta k k^T) Diag(alpha)."""
    outs, finals = [], []
    H, dk = q.shape[2], q.shape[3]
    I = torch.eye(dk, dtype=torch.float64)
    for n in range(len(starts) - 1):
        o_n, f_n = [], []
        for h in range(H):
            S = S0[n, h]
            o_h = []
            for t in range(int(starts[n]), int(starts[n + 1])):
                M = (I - beta[0, t, h] * torch.outer(k[0, t, h], k[0, t, h])) @ torch.diag(torch.exp(la[0, t, h]))
                S = M @ S + beta[0, t, h] * torch.outer(k[0, t, h], v[0, t, h])
                o_h.append(S.T @ q[0, t, h])
            o_n.append(torch.stack(o_h))
            f_n.append(S)
        outs.append(torch.stack(o_n, dim=1))
        finals.append(torch.stack(f_n))
    return torch.cat(outs, dim=0), torch.stack(finals)


def test_gradients_match_torch_autograd_across_checkpoint_segments():
    rng = np.random.default_rng(11)
    dk = dv = 16
    H = 2
    starts = np.array([0, 70, 135])  # both sequences longer than one 64-token checkpoint segment
    T = int(starts[-1])
    q, k, v, la, beta = _inputs(rng, 1, T, H, dk, dv, decay=0.2)
    S0 = rng.standard_normal((2, H, dk, dv)) * 0.1
    do = rng.standard_normal((1, T, H, dv)).astype(np.float32)
    dfin = rng.standard_normal((2, H, dk, dv))
    g = oracle.backward(q, k, v, la, beta, d_o=do, initial_state=S0, d_final=dfin, cu_seqlens=starts)

    tt = {n: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
          for n, a in (("q", q), ("k", k), ("v", v), ("la", la), ("beta", beta), ("S0", S0))}
    o, fin = _torch_recurrence(tt["q"], tt["k"], tt["v"], tt["la"], tt["beta"], tt["S0"], starts)
    L = (o * torch.tensor(do[0], dtype=torch.float64)).sum() + (fin * torch.tensor(dfin)).sum()
    L.backward()
    pairs = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("la", "dlog_alpha"), ("beta", "dbeta"), ("S0", "d_initial"))
    for tn, on in pairs:
        ref = tt[tn].grad.numpy()
        err = np.abs(g[on] - ref).max() / max(np.abs(ref).max(), 1e-30)
        assert err < 1e-11, (on, err)


def test_chain_rule_across_a_split_sequence():
    """Backward over tokens [0, T) equals backward over [s, T) followed by backward
    over [0, s) with the first part's initial-state gradient as the final-state
    cotangent (and the forward state at s as the second part's initial state)."""
    rng = np.random.default_rng(4)
    T, H, d, s = 90, 2, 8, 37
    q, k, v, la, beta = _inputs(rng, 1, T, H, d, d)
    S0 = rng.standard_normal((1, H, d, d))
    do = rng.standard_normal((1, T, H, d)).astype(np.float32)
    dfin = rng.standard_normal((1, H, d, d))
    full = oracle.backward(q, k, v, la, beta, d_o=do, initial_state=S0, d_final=dfin)
    _, S_mid = oracle.forward(q[:, :s], k[:, :s], v[:, :s], la[:, :s], beta[:, :s], initial_state=S0,
                              want_o=False)
    g2 = oracle.backward(q[:, s:], k[:, s:], v[:, s:], la[:, s:], beta[:, s:], d_o=do[:, s:], initial_state=S_mid,
                         d_final=dfin)
    g1 = oracle.backward(q[:, :s], k[:, :s], v[:, :s], la[:, :s], beta[:, :s], d_o=do[:, :s], initial_state=S0,
                         d_final=g2["d_initial"])
    for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
        joined = np.concatenate([g1[name], g2[name]], axis=1)
        assert np.allclose(joined, full[name], rtol=1e-10, atol=1e-12), name
    assert np.allclose(g1["d_initial"], full["d_initial"], rtol=1e-10, atol=1e-12)


def test_gradients_are_linear_in_the_cotangents():
    rng = np.random.default_rng(8)
    T, H, d = 20, 1, 8
    q, k, v, la, beta = _inputs(rng, 1, T, H, d, d)
    # quarter-integers: the float32 sum do1 + do2 that the C oracle receives is exact
    do1 = (rng.integers(-8, 9, (1, T, H, d)) / 4).astype(np.float32)
    do2 = (rng.integers(-8, 9, (1, T, H, d)) / 4).astype(np.float32)
    f1 = rng.standard_normal((1, H, d, d))
    f2 = rng.standard_normal((1, H, d, d))
    g1 = oracle.backward(q, k, v, la, beta, d_o=do1, d_final=f1)
    g2 = oracle.backward(q, k, v, la, beta, d_o=do2, d_final=f2)
    g12 = oracle.backward(q, k, v, la, beta, d_o=(do1 + do2), d_final=f1 + f2)
    for name in g1:
        assert np.allclose(g12[name], g1[name] + g2[name], rtol=1e-9, atol=1e-11), name


def test_zero_length_sequence_passes_the_cotangent_through():
    rng = np.random.default_rng(1)
    H, d = 2, 4
    q, k, v, la, beta = _inputs(rng, 1, 3, H, d, d)
    dfin = rng.standard_normal((2, H, d, d))
    g = oracle.backward(q, k, v, la, beta, d_final=dfin, cu_seqlens=[0, 0, 3])
    assert np.array_equal(g["d_initial"][0], dfin[0])


BWD_MUTANTS = {
    "de_without_beta": ("de[j] = b * r[j];", "de[j] = r[j];"),
    "dbeta_with_do": ("db += r[j] * e[j];", "db += r[j] * dov[j];"),
    "dk_read_sign": ("dk_out[rk + i] -= acc;", "dk_out[rk + i] += acc;"),
    "carry_without_decay": ("L[(size_t)i * dv + j] = alpha[i] * dSp[(size_t)i * dv + j];",
                            "L[(size_t)i * dv + j] = dSp[(size_t)i * dv + j];"),
    "dq_from_old_state": ("acc += St[(size_t)i * dv + j] * dov[j];", "acc += Sprev[(size_t)i * dv + j] * dov[j];"),
    "dsp_sign": ("dSp[(size_t)i * dv + j] = L[(size_t)i * dv + j] - kt[i] * de[j];",
                 "dSp[(size_t)i * dv + j] = L[(size_t)i * dv + j] + kt[i] * de[j];"),
    "dlog_alpha_unscaled": ("dlog_alpha[rk + i] = alpha[i] * acc;", "dlog_alpha[rk + i] = acc;"),
    "output_cotangent_on_k": ("L[(size_t)i * dv + j] += qt[i] * dov[j];", "L[(size_t)i * dv + j] += kt[i] * dov[j];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_planted_backward_mistakes_fail_the_pin(tmp_path, name):
    a, b = BWD_MUTANTS[name]
    text = open(SRC).read()
    assert text.count(a) == 1, name
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(text.replace(a, b))
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    assert fd_failures(lib=oracle.load_library(str(so))) != []
