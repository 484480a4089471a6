"""Pins for the oracle's output head and flow mixture (CPU only)."""
import numpy as np
import torch

import dfx_inputs as gen
from oracle.head import mixture, next_token, output_head, softmax
from oracle.linear import grouped_linear, rmsnorm
from oracle.numerics import widen


def test_softmax_matches_torch():
    z = np.random.default_rng(1).standard_normal((3, 50)) * 4
    assert np.allclose(softmax(z), torch.softmax(torch.from_numpy(z), dim=-1).numpy(), rtol=0, atol=1e-15)


def test_mixture_properties():
    rng = np.random.default_rng(2)
    p1, p2 = softmax(rng.standard_normal((4, 30)) * 3), softmax(rng.standard_normal((4, 30)))
    alpha, c, pm = mixture(p1, p2)
    assert np.all((alpha >= 0.5) & (alpha <= 1.0))
    assert np.allclose(pm.sum(-1), 1.0, atol=1e-14)
    # a certain primary takes the whole weight; a flat one (c = 1/V) the least
    onehot = np.eye(30)[[3, 7, 0, 29]]
    a1, _, pm1 = mixture(onehot, p2)
    assert np.array_equal(a1, np.ones(4)) and np.array_equal(pm1, onehot)
    flat = np.full((4, 30), 1 / 30)
    a0, c0, _ = mixture(flat, p2)
    assert np.allclose(c0, 1 / 30, atol=1e-15) and np.allclose(a0, 0.5 * (1 + 1 / 30), atol=1e-15)
    # alpha grows with the primary's confidence
    sharp = softmax(np.log(p1) * 3)
    assert np.all(mixture(sharp, p2)[0] > alpha)
    # primary alone: p_mix is the primary's distribution
    a, _, pm = mixture(p1)
    assert np.array_equal(pm, p1) and np.all(a == 1)


def test_greedy_and_gumbel_max():
    rng = np.random.default_rng(3)
    p = softmax(rng.standard_normal((5, 40)) * 2)
    assert np.array_equal(next_token(p), torch.argmax(torch.from_numpy(p), dim=-1).numpy())
    # Gumbel-max with many independent noise draws samples p: empirical frequencies vs p
    n = 40000
    u = rng.uniform(size=(n, 40))
    counts = np.bincount(next_token(np.repeat(p[:1], n, axis=0), u), minlength=40) / n
    assert np.max(np.abs(counts - p[0])) < 0.012


def test_output_head_composes_norm_projection_and_mixture():
    rng = np.random.default_rng(4)
    V, H = 48, 64
    x = rng.standard_normal((2, 3, H)).astype(np.float32)
    g = rng.uniform(0.9, 1.1, H).astype(np.float32)
    w = gen.f32_to_bf16_bits(rng.standard_normal((V, H)).astype(np.float32) * 0.1)
    tok, alpha, pm, mid = output_head(x, g, 1e-5, w)
    h = rmsnorm(x, g, 1e-5)
    logits = torch.nn.functional.linear(torch.from_numpy(h), torch.from_numpy(widen(w))).numpy()
    assert np.allclose(mid["logits"], logits, rtol=0, atol=1e-12)
    p = torch.softmax(torch.from_numpy(logits), dim=-1).numpy()
    c = (p[0] ** 2).sum(-1)
    assert np.allclose(alpha, (1 + c) / 2, atol=1e-14)
    assert np.allclose(pm, alpha[:, None] * p[0] + (1 - alpha[:, None]) * p[1], atol=1e-14)
    assert np.array_equal(tok, pm.argmax(-1))
