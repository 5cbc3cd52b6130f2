"""Planted mistakes in copies of the oracle must fail its pins (CPU only).

Each mutant is the oracle's C source with one plausible mistake (a dropped term,
a wrong sign, a wrong index, a swapped operand), compiled into a temporary
library. The pins of ``test_oracle_pins.py`` -- the hand-worked example, the dense
transition product, the DeltaNet and Gated DeltaNet reductions and exact
retrieval -- are run against it; at least one must reject it. The unmodified
source passes all of them.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import reference

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "kda_oracle.c")

MUTANTS = {
    "decay_dropped": ("S[(size_t)i * w + j] *= alpha[i];", "(void)alpha;"),
    "delta_sign": ("e[j] = (double)v[rv + c0 + j] - e[j];", "e[j] = (double)v[rv + c0 + j] + e[j];"),
    "beta_dropped": ("const double bki = b * kt[i];", "const double bki = kt[i]; (void)b;"),
    "decay_channel_shift": (": (double)log_alpha[i];", ": (double)log_alpha[(i + 1) % dk];"),
    "read_with_q": ("const double ki = kt[i];", "const double ki = qt[i];"),
    "output_with_k": ("const double qi = qt[i];", "const double qi = kt[i];"),
    "decay_exponent": ("alpha[i] = exp(la);", "alpha[i] = exp(0.5 * la);"),
}


def build_variant(tmp_path, name, text):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(text)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    return oracle.load_library(str(so))


def pins_pass(lib):
    """Runs the pins against ``lib``; returns the names of those that fail."""
    failed = []
    rng = np.random.default_rng(5)
    # hand-worked example
    with open(os.path.join(HERE, "golden", "hand_worked_d2.json")) as f:
        g = json.load(f)
    x = g["inputs"]
    o, S = oracle.forward(np.array(x["q"])[None, :, None], np.array(x["k"])[None, :, None],
                          np.array(x["v"])[None, :, None], np.log(np.array(x["alpha"]))[None, :, None],
                          np.array(x["beta"])[None, :, None], np.array(x["initial_state"])[None, None], lib=lib)
    if not (np.allclose(o[0, :, 0], g["expected"]["o"], atol=1e-7) and
            np.allclose(S[0, 0], g["expected"]["final_state"], atol=1e-7)):
        failed.append("hand_worked")
    # dense transition product
    T, dk, dv = 6, 5, 4
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, dv))
    la = -0.5 * rng.random((T, dk))
    beta = rng.random(T)
    S0 = rng.standard_normal((dk, dv))
    f32 = lambda a: a.astype(np.float32)
    q, k, v, la, beta = map(f32, (q, k, v, la, beta))
    o, S = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None], la[None, :, None],
                          beta[None, :, None], S0[None, None], lib=lib)
    o_ref, S_ref = reference.dense_closed_form(q, k, v, la, beta, S0)
    if not (np.allclose(o[0, :, 0], o_ref, atol=1e-10) and np.allclose(S[0, 0], S_ref, atol=1e-10)):
        failed.append("dense")
    # DeltaNet reduction
    o, S = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None], np.zeros_like(la)[None, :, None],
                          beta[None, :, None], S0[None, None], lib=lib)
    o_ref, S_ref = reference.deltanet(q, k, v, beta, S0)
    if not (np.allclose(o[0, :, 0], o_ref, atol=1e-10) and np.allclose(S[0, 0], S_ref, atol=1e-10)):
        failed.append("deltanet")
    # Gated DeltaNet reduction
    gate = f32(-0.3 * rng.random(T))
    la_s = np.repeat(gate[:, None], dk, axis=1)
    o, S = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None], la_s[None, :, None],
                          beta[None, :, None], S0[None, None], lib=lib)
    o_ref, S_ref = reference.gated_deltanet(q, k, v, gate, beta, S0)
    if not (np.allclose(o[0, :, 0], o_ref, atol=1e-10) and np.allclose(S[0, 0], S_ref, atol=1e-10)):
        failed.append("gdn")
    # exact retrieval with beta = 1 and q = k
    o, _ = oracle.forward(k[None, :, None], k[None, :, None], v[None, :, None], la[None, :, None],
                          np.ones_like(beta)[None, :, None], S0[None, None], lib=lib)
    if not np.allclose(o[0, :, 0], v, atol=1e-5):
        failed.append("retrieval")
    return failed


def test_unmodified_source_passes(tmp_path):
    lib = build_variant(tmp_path, "orig", open(SRC).read())
    assert pins_pass(lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    lib = build_variant(tmp_path, name, src.replace(old, new))
    failed = pins_pass(lib)
    assert failed, f"mutant {name} passed every pin"
