"""The seeded input generator (gated_delta_rule_57_amd/inputs.py) against its stated
recipe, on the CPU: values rebuilt from SeedSequence and default_rng by hand, the
independence of the values from the number of filling threads, and the structure of
each recipe (mixed slow channels, packed lengths, the tied DPLR pair)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_57_amd import inputs


def _unit_rows(x, d=128):
    x = x.reshape(-1, d)
    return (x / np.sqrt(np.sum(x * x, axis=1, keepdims=True))).ravel()


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def test_prefill_values_follow_the_recipe():
    """q, k, v, decays and beta of a small prefill, rebuilt draw by draw: each draw is
    the next child of SeedSequence(seed), its one block the child's first child."""
    seed, T, H = 5, 7, 2
    inp = inputs.make_prefill(seed, B=1, T=T, H=H, dtype="bf16", la_scale=0.3, s0_std=0.02, device="cpu")
    root = np.random.SeedSequence(seed)
    draw = lambda n, fn: fn(np.random.default_rng(root.spawn(1)[0].spawn(1)[0]), n)  # noqa: E731
    nk = T * H * 128
    q = draw(nk, lambda r, n: _unit_rows(r.standard_normal(n)))
    k = draw(nk, lambda r, n: _unit_rows(r.standard_normal(n)))
    v = draw(nk, lambda r, n: r.standard_normal(n))
    la = draw(nk, lambda r, n: -0.3 * np.logaddexp(0.0, r.standard_normal(n)))
    beta = draw(T * H, lambda r, n: 1.0 / (1.0 + np.exp(-r.standard_normal(n))))
    s0 = draw(H * 128 * 128, lambda r, n: 0.02 * r.standard_normal(n))
    got = inp.numpy()
    assert np.array_equal(got["q"].ravel(), _bf16(q))
    assert np.array_equal(got["k"].ravel(), _bf16(k))
    assert np.array_equal(got["v"].ravel(), _bf16(v))
    assert np.array_equal(got["log_alpha"].ravel(), la.astype(np.float32))
    assert np.array_equal(got["beta"].ravel(), beta.astype(np.float32))
    assert np.array_equal(got["initial_state"].ravel(), s0.astype(np.float32))


def test_values_do_not_depend_on_thread_count(monkeypatch):
    """A draw of several blocks is the same filled by one thread or by several."""
    monkeypatch.setattr(inputs, "BLOCK", 1024)
    outs = []
    for n in (1, 3):
        monkeypatch.setattr(inputs, "_host_threads", lambda n=n: n)
        outs.append(inputs.HostDraws(11).fill(5000, lambda r, c: r.standard_normal(c)))
    assert np.array_equal(outs[0], outs[1])
    # block b comes from the b-th child of the draw's child
    kid = np.random.SeedSequence(11).spawn(1)[0]
    b2 = np.random.default_rng(kid.spawn(5)[2]).standard_normal(1024).astype(np.float32)
    assert np.array_equal(outs[0][2048:3072], b2)


def test_mixed_decays_have_half_slow_channels():
    inp = inputs.make_prefill(3, B=1, T=40, H=4, dtype="bf16", la_mode="mixed", device="cpu")
    la = inp.log_alpha.numpy()[0]  # [T, H, 128]
    for h in range(4):
        slow = np.all(la[:, h, :] == np.float32(-1e-3), axis=0)
        assert slow.sum() == 64
        assert np.all(la[:, h, ~slow] < 0)


def test_packed_lengths_are_a_composition():
    inp = inputs.make_prefill(2, B=1, T=1000, H=1, dtype="bf16", num_seqs=7, device="cpu")
    cu = inp.cu_seqlens.numpy()
    assert cu[0] == 0 and cu[-1] == 1000 and len(cu) == 8
    assert np.all(np.diff(cu) > 0)


def test_raw_and_cotangent_draws_are_seeded():
    a = inputs.make_raw_prefill(4, B=1, T=30, H=2, dtype="bf16", num_seqs=3, s0_std=0.1, device="cpu")
    b = inputs.make_raw_prefill(4, B=1, T=30, H=2, dtype="bf16", num_seqs=3, s0_std=0.1, device="cpu")
    for x, y in zip(a.numpy().values(), b.numpy().values()):
        assert (x is None and y is None) or np.array_equal(x, y)
    w = a.norm_weight.numpy()
    assert np.all((w >= 0.5) & (w < 1.5))
    inp = inputs.make_prefill(4, B=1, T=30, H=2, dtype="bf16", device="cpu")
    g1, f1 = inputs.make_cotangents(4, inp, device="cpu")
    g2, f2 = inputs.make_cotangents(4, inp, device="cpu")
    assert torch.equal(g1, g2) and torch.equal(f1, f2)
    assert g1.dtype == torch.bfloat16 and f1.shape == (1, 2, 128, 128)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tied_dplr_pair_is_exact(dtype):
    """a = -2^-j b with j >= 1, exactly in the compute dtype."""
    x = inputs.make_dplr(9, B=1, T=50, H=2, dtype=dtype, device="cpu")
    a, b = x.a.double().numpy(), x.b.double().numpy()
    ratio = np.where(b != 0, a / np.where(b != 0, b, 1), np.nan)
    r = np.nanmax(ratio, axis=-1)
    assert np.allclose(np.nanmin(ratio, axis=-1), r)  # one ratio per (token, head)
    j = -np.log2(-r)
    assert np.all(j >= 1) and np.array_equal(j, np.round(j))
