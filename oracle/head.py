"""Shared output head and the mixture of the two flows' predictions (oracle, fp64).

What is computed (Sintesi Tecnica: Dual-Flow Transformers, "Architettura Core": both flows
share the output matrix; "Meccanismi Chiave", mixture objective): each flow's final residual
row is normalized (one gain vector for both) and projected by the one shared vocabulary
matrix; each flow's logits give a softmax distribution, and the prediction is
p_mix = alpha_t p_primary + (1 - alpha_t) p_aux, with alpha_t driven by the primary's
confidence -- its collision probability c_t = sum_i p_primary,i^2 -- and never below 1/2.

Reading (the pages give no formula for alpha_t): alpha_t = (1 + c_t) / 2, the plainest map
that is monotone in the collision probability, equals 1/2 only as c_t -> 0 and 1 when the
primary is certain. Parity of this formula is unpinned beyond those stated properties.
Rounding point R6: the normed rows are rounded to bf16 before the projection, as every row
entering a shared matrix is. The next token is argmax_i p_mix,i (lowest index on ties), or,
with uniform noise u in (0, 1), argmax_i (log p_mix,i - log(-log u_i)): a Gumbel-max draw from
p_mix, the noise being an input.
"""
import numpy as np

from .linear import grouped_linear, rmsnorm


def softmax(logits):
    z = np.asarray(logits, np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def mixture(p_primary, p_aux=None):
    """(alpha [B], collision [B], p_mix [B][V]) from the flows' distributions."""
    c = np.sum(p_primary * p_primary, axis=-1)
    if p_aux is None:
        return np.ones_like(c), c, p_primary
    alpha = 0.5 * (1.0 + c)
    return alpha, c, alpha[:, None] * p_primary + (1.0 - alpha[:, None]) * p_aux


def next_token(p_mix, uniform_noise=None):
    if uniform_noise is None:
        return np.argmax(p_mix, axis=-1).astype(np.int32)
    with np.errstate(divide="ignore"):
        score = np.log(p_mix) - np.log(-np.log(np.asarray(uniform_noise, np.float64)))
    return np.argmax(score, axis=-1).astype(np.int32)


def output_head(x, gain, eps, w_out, uniform_noise=None):
    """x: float [F][B][hidden] final residual rows; w_out: uint16 bf16 [vocab][hidden].
    Returns (tokens [B], alpha [B], p_mix [B][V], dict of intermediates)."""
    h = rmsnorm(x, gain, eps)                                   # R6
    logits = grouped_linear(h, w_out)                           # [F][B][V]
    p = softmax(logits)
    alpha, c, p_mix = mixture(p[0], p[1] if p.shape[0] == 2 else None)
    return next_token(p_mix, uniform_noise), alpha, p_mix, dict(h=h, logits=logits, p=p, collision=c)
