"""Mixture-of-experts MLP with router replay (oracle, fp64).

What is computed (Sintesi Tecnica: Dual-Flow Transformers, "Meccanismi Chiave", router
replay: in an MoE model the auxiliary flow takes the experts that the primary's router chose
and combines them with mixture weights of its own; "Contributi Chiave" item 3 and the
closing section: the two flows' expert fan-outs are independent settings, the decode cost
being the sum of both flows' expert use).

Readings (the pages give no formula):
  - one router matrix W_r [E][hidden], shared like every other matrix, scores each flow's
    normed row: logits_f = h_f W_r^T;
  - the ranking is the primary's logits in descending order, the lower expert id first on
    equal logits; the primary takes the first k1 experts of it, the auxiliary the first k2
    of the same ranking (k2 below k1 is a subset of the primary's experts, above it the
    ranking continues past them);
  - a flow's mixture weights are the softmax of its own logits over its selected experts;
  - expert e is a SwiGLU MLP with its own W_gate_up[e] [2I][hidden] and W_down[e] [hidden][I];
  - coupling b acts on each expert's intermediate, inter_aux,e += b * inter_prim,e, where
    inter_prim,e is the primary's intermediate of e if the primary selected e, else zero;
    coupling c acts on the block output, mlp_aux += c * mlp_prim, before the residual add;
  - bf16 rounding points: the normed rows (as before every shared matrix) and each expert's
    intermediate (as the dense MLP's); a flow's expert outputs are added in ranking order.
"""
import numpy as np

from .linear import rmsnorm
from .numerics import round_bf16, widen


def ranking(logits_primary):
    """Expert ids of each row by descending primary logit, lower id first on ties."""
    lp = np.asarray(logits_primary, np.float64)
    return np.argsort(-lp, axis=-1, kind="stable")


def route(logits, k1, k2):
    """logits: [F][B][E]. Returns ids (list per flow of int [B][k_f]) and weights (list per
    flow of float64 [B][k_f]) -- the primary's top-k1 and the same ranking's top-k2 for the
    auxiliary, each weighted by the softmax of its own logits over its experts."""
    order = ranking(logits[0])
    ids, weights = [], []
    for f in range(logits.shape[0]):
        sel = order[:, : (k1 if f == 0 else k2)]
        z = np.take_along_axis(np.asarray(logits[f], np.float64), sel, axis=-1)
        e = np.exp(z - z.max(axis=-1, keepdims=True))
        ids.append(sel)
        weights.append(e / e.sum(axis=-1, keepdims=True))
    return ids, weights


def expert_intermediate(h, w_gate_up_e):
    """silu(h W_g^T) * (h W_u^T) for one expert, before the bf16 rounding; h: [..][hidden]."""
    gu = widen(h) @ widen(w_gate_up_e).T
    I = gu.shape[-1] // 2
    g, u = gu[..., :I], gu[..., I:]
    return g / (1.0 + np.exp(-g)) * u


def moe_mlp(x, gain, eps, w_router, w_gate_up, w_down, k1, k2, b=None, c=None, selection=None):
    """x: float [F][B][hidden] residual rows; w_router uint16 [E][hidden]; w_gate_up uint16
    [E][2I][hidden]; w_down uint16 [E][hidden][I]; b [I], c [hidden] or None.

    selection: optional (ids, weights) replacing the routing (a kernel's own decisions), so
    that everything after the top-k choice can be compared on the same experts.
    Returns (x_out fp64 [F][B][hidden], dict of intermediates)."""
    x = np.asarray(x, np.float64)
    F, B, H = x.shape
    h = rmsnorm(x, gain, eps)                                    # bf16 values
    logits = widen(h) @ widen(w_router).T                        # [F][B][E]
    ids, weights = route(logits, k1, k2) if selection is None else selection
    out = np.zeros((F, B, H))
    inter_all = {}
    for bb in range(B):
        prim_inter = {}
        for f in range(F):
            for j, e in enumerate(ids[f][bb]):
                e = int(e)
                inter = expert_intermediate(h[f, bb], w_gate_up[e])
                if f == 0:
                    prim_inter[e] = inter
                elif b is not None:
                    inter = inter + widen(b) * prim_inter.get(e, 0.0)
                inter = round_bf16(inter)
                inter_all[(f, bb, e)] = inter
                out[f, bb] += weights[f][bb, j] * (inter @ widen(w_down[e]).T)
    if c is not None and F == 2:
        out[1] = out[1] + widen(c) * out[0]
    return x + out, dict(h=h, logits=logits, ids=ids, weights=weights, inter=inter_all, mlp=out)
