"""GPU parity of the shared output head and flow mixture (dfx_dual_flow_output_head).

Checked as a chain, each stage against the oracle applied to the GPU's own previous stage
(read from the workspace): the bf16 normed rows (rounding decisions), the fp32 logits
(accumulation bound), then p_mix, alpha and the token from the GPU's logits (fp32 softmax
bounds), and the token as the exact arg max of the GPU's own p_mix."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
import dual_flow_shared_amd as dfx
from gpu_util import bf16_decisions_agree, dev, unpack_rows
from oracle.head import mixture, output_head, softmax
from oracle.linear import rmsnorm
from oracle.numerics import widen

pytestmark = pytest.mark.gpu

U = 2.0 ** -24                 # fp32 unit roundoff
TINY = 2.0 ** -126             # probabilities below the fp32 normal range may flush to zero


def gamma(k):
    """Accumulation bound of a k-term fp32 dot product on the matrix cores (32-term blocks
    added over k / 32 steps, plus split-K partial sums)."""
    return (k / 32 + 64) * U


def run(c, F, noise=False, want_p=True, w_packed=None):
    B, H = c.x.shape[1], c.x.shape[2]
    V = c.w_out.shape[0]
    w = dfx.pack_weight(dev(c.w_out)) if w_packed is None else w_packed
    ws = dfx.Workspace()
    tok, alpha, pm = dfx.output_head(dev(c.x[:F].copy()), dev(c.gain), c.eps, w,
                                     dev(c.noise) if noise else None, want_p_mix=want_p, workspace=ws)
    torch.cuda.synchronize()
    taps = dfx.output_head_taps(F, B, H, V)
    buf = ws.buf.cpu().numpy()
    padded = -(-B // (64 // F)) * 64
    h = unpack_rows(buf[taps["h"]: taps["h"] + padded * H * 2].view(np.uint16), F, B, H)
    logits = buf[taps["logits"]: taps["logits"] + F * B * V * 4].view(np.float32).reshape(F, B, V)
    return (tok.cpu().numpy(), alpha.cpu().numpy().astype(np.float64),
            None if pm is None else pm.cpu().numpy(), h, logits.astype(np.float64), w)


def check_norm(c, F, h):
    """R6: the GPU's bf16 normed rows are roundings of values within the fp32 norm's error of
    the exact ones."""
    H = c.x.shape[2]
    x = c.x[:F].astype(np.float64)
    exact = rmsnorm(x, c.gain, c.eps, rounded=False)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + c.eps)
    scale = np.abs(c.gain.astype(np.float64)) * r * np.abs(x) * (H / 2 + 8) * U + 4 * U * np.abs(exact)
    return bf16_decisions_agree(h, exact, rel=1.0, scale=scale)


def check_logits(c, h, logits, cols=None):
    """fp32 logits within the accumulation bound of the fp64 projection of the GPU's h."""
    H = h.shape[-1]
    w = c.w_out if cols is None else c.w_out[cols]
    ref = widen(h) @ widen(w).T
    bound = gamma(H) * (np.abs(widen(h)) @ np.abs(widen(w)).T) + 1e-30
    got = logits if cols is None else logits[..., cols]
    assert np.all(np.abs(got - ref) <= bound)


def mixture_bounds(logits):
    """Oracle mixture of the GPU's logits, and per-element error bounds of the fp32 kernels:
    the shifted logit l - m rounds (|l - m| U), exp, the chunked sums (<= 2 kMixRounds + tree
    levels + chunk combination, under 200 U), the weights alpha / s and (1 - alpha) / s, and
    alpha from q / s^2 (under 400 U relative in the collision probability)."""
    p = softmax(logits)
    F = logits.shape[0]
    alpha, coll, pm = mixture(p[0], p[1] if F == 2 else None)
    d = np.abs(logits - logits.max(axis=-1, keepdims=True))
    rel = (d + 200) * U
    dalpha = 400 * U * coll + 2 * U
    if F == 2:
        tol = (alpha[:, None] * p[0] * rel[0] + (1 - alpha[:, None]) * p[1] * rel[1]
               + dalpha[:, None] * np.abs(p[0] - p[1]) + 2 * U * pm)
    else:
        tol = p[0] * rel[0] + 2 * U * pm
        dalpha = np.zeros_like(alpha)
    return alpha, pm, tol + 2 * TINY, dalpha


def check_mixture(logits, tok, alpha, pm, noise=None):
    a_ref, pm_ref, tol, da = mixture_bounds(logits)
    assert np.all(np.abs(alpha - a_ref) <= da + 1e-30)
    if pm is not None:
        assert np.all(np.abs(pm.astype(np.float64) - pm_ref) <= tol)
    rows = np.arange(len(tok))
    if noise is None:
        # the token is a maximum of the oracle's p_mix up to the bounds of the two candidates
        best = pm_ref.argmax(-1)
        assert np.all(pm_ref[rows, tok] + tol[rows, tok] >= pm_ref[rows, best] - tol[rows, best])
        if pm is not None:
            assert np.array_equal(tok, pm.argmax(-1))           # first maximum of the GPU's p_mix
    else:
        u = noise.astype(np.float64)
        with np.errstate(divide="ignore"):
            g = -np.log(-np.log(u))
            score = np.log(pm_ref) + g
        # fp32 logs: one rounding per log on top of p_mix's own bound
        stol = tol / np.maximum(pm_ref, TINY) + 4 * U * (np.abs(np.log(np.maximum(pm_ref, TINY))) + np.abs(g) + 2)
        best = score.argmax(-1)
        assert np.all(score[rows, tok] + stol[rows, tok] >= score[rows, best] - stol[rows, best])
    return float(np.mean(tok == (pm_ref.argmax(-1) if noise is None else best)))


@pytest.mark.parametrize("F", [2, 1])
# (batch, hidden, vocab): the first three project in one K split (output-head mode, two 128-logit
# tiles per work-group) over an odd tile count (9, 157, 1), so the last work-group's second tile
# lies past the vocabulary; the fourth splits K (separate statistics pass)
@pytest.mark.parametrize("shape", [(3, 256, 1040), (40, 512, 20016), (5, 256, 48), (3, 4096, 1040)])
def test_head_chain_small(F, shape):
    B, H, V = shape
    c = gen.head_case(900 + B, 2, B, H, V, w_std=0.4)
    tok, alpha, pm, h, logits, w = run(c, F)
    check_norm(c, F, h)
    check_logits(c, h, logits)
    check_mixture(logits, tok, alpha, pm)
    if F == 1:
        assert np.all(alpha == 1.0)
    else:
        assert np.all((alpha >= 0.5) & (alpha <= 1.0)) and alpha.std() > 0.01   # distinct confidences
    # the same call without p_mix returns the same token and alpha
    tok2, alpha2, pm2, _, _, _ = run(c, F, want_p=False, w_packed=w)
    assert pm2 is None and np.array_equal(tok2, tok) and np.array_equal(alpha2, alpha)
    # end to end against the oracle from x (bf16 rounding decisions of h may differ slightly)
    _, a_or, pm_or, _ = output_head(c.x[:F], c.gain, c.eps, c.w_out)
    assert np.max(np.abs(pm - pm_or)) < 5e-2 * pm_or.max() and np.max(np.abs(alpha - a_or)) < 1e-2


@pytest.mark.parametrize("F", [2, 1])
def test_head_gumbel_max(F):
    c = gen.head_case(911, 2, 40, 256, 20016, w_std=0.3)
    tok, alpha, pm, h, logits, _ = run(c, F, noise=True)
    check_logits(c, h, logits)
    agree = check_mixture(logits, tok, alpha, pm, noise=c.noise)
    assert agree > 0.9
    greedy = pm.argmax(-1)
    assert np.any(tok != greedy)               # the draw is not the greedy choice everywhere


def test_head_flat_distribution_ties_to_lowest_index():
    """All logits zero (W_out = 0): p is uniform, c = 1 / V, alpha = (1 + 1 / V) / 2 and every
    token ties, so the token is 0."""
    c = gen.head_case(912, 2, 5, 64, 4096)
    c.w_out[:] = 0
    tok, alpha, pm, _, logits, _ = run(c, 2)
    assert np.all(logits == 0) and np.all(tok == 0)
    assert np.allclose(alpha, 0.5 * (1 + 1 / 4096), rtol=0, atol=4 * U)
    assert np.allclose(pm, 1 / 4096, rtol=8 * U, atol=0)


def test_head_empty_batch():
    c = gen.head_case(913, 2, 1, 64, 64)
    x = torch.empty(2, 0, 64, device="cuda")
    tok, alpha, pm = dfx.output_head(x, dev(c.gain), c.eps, dfx.pack_weight(dev(c.w_out)), want_p_mix=True)
    torch.cuda.synchronize()
    assert tok.numel() == 0 and alpha.numel() == 0 and pm.shape == (0, 64)


def test_head_full_size_sampled():
    """hidden 4096 and a 128256-token vocabulary at batch 32, both flows: every normed row,
    logits on sampled columns (and each row's winner), the mixture on all columns."""
    c = gen.head_case(914, 2, 32, 4096, 128256)
    tok, alpha, pm, h, logits, _ = run(c, 2)
    check_norm(c, 2, h)
    cols = np.unique(np.concatenate([np.random.default_rng(5).choice(128256, 1024, replace=False),
                                     tok, np.arange(8), np.arange(128256 - 8, 128256)]))
    check_logits(c, h, logits, cols)
    check_mixture(logits, tok, alpha, pm)


def test_head_smallest_vocabulary():
    """vocab 16: one 16-wide projection tile, one partial mixture chunk."""
    c = gen.head_case(915, 2, 3, 64, 16, w_std=0.5)
    tok, alpha, pm, h, logits, _ = run(c, 2)
    check_logits(c, h, logits)
    check_mixture(logits, tok, alpha, pm)
    assert np.allclose(pm.sum(-1), 1.0, atol=1e-5)
