"""Dual-query decode attention over the primary flow's K/V cache (oracle, fp64).

What is computed (Sintesi Tecnica: Dual-Flow Transformers, "Meccanismi
Chiave", asymmetric shared-KV attention): the primary query Q1 attends to the
primary keys and values K1, V1 as in ordinary causal self-attention; the
auxiliary flow forms its own query Q2, coupled to Q1 through a learned vector
a, and attends to the same K1, V1; the auxiliary flow writes no cache.

Readings of what the pages leave open:
  * coupling: Q2 = q2_raw + a * Q1 elementwise, where q2_raw = Wq x2 is the
    auxiliary row's own projection; a is one vector per layer of length
    head_dim (a_head_stride 0) or one per query head (a_head_stride = D);
  * scores s_p = scale * <Q, K_p> with scale = 1 / sqrt(D) for both flows;
  * grouped-query heads: query head h reads KV head h // (Hq / Hkv);
  * both flows attend to positions [0, ctx_b) of sequence b (the primary's
    current token already appended); ctx_b = 0 gives O = 0 and lse = -inf;
  * softmax weights w = exp(s - max s) / sum exp(s - max s),
    O = sum_p w_p V_p, lse = max s + log sum exp(s - max s).
Cache addressing: position p of sequence b, KV head g lives at
pool[blk][g][p % block_size] with blk = block_table[b][p // block_size];
without a table, sequence b owns pool[b] and block_size is its capacity.
"""
import math

import numpy as np

from .numerics import widen


def _queries(q1, q2_raw, a, a_head_stride, dtype=np.float64):
    Q1 = widen(q1).astype(dtype)
    B, Hq, D = Q1.shape
    flows = [Q1]
    if q2_raw is not None:
        Q2 = widen(q2_raw).astype(dtype)
        if a is not None:
            A = widen(a).astype(dtype)
            A = A.reshape(1, 1, D) if a_head_stride == 0 else A.reshape(1, Hq, D)
            Q2 = Q2 + A * Q1
        flows.append(Q2)
    return flows


def gather_kv(pool, block_table, b, n):
    """Logical rows [Hkv][n][D] of sequence b, gathered through the table (no arithmetic)."""
    if block_table is None:
        return pool[b, :, :n, :]
    bs = pool.shape[2]
    p = np.arange(n)
    blk = np.asarray(block_table)[b, p // bs]
    return np.transpose(pool[blk, :, p % bs, :], (1, 0, 2))


def decode_attention(q1, q2_raw, a, a_head_stride, k_pool, v_pool, block_table, context_lens,
                     softmax_scale=None, batches=None, return_weights=False, dtype=np.float64):
    """Dual-flow decode attention in fp64.

    q1, q2_raw: [B][Hq][D] (uint16 bf16 bits, float32 or float64); q2_raw may be
    None (primary only). a: [D] or [Hq][D] or None. Pools: [blocks][Hkv][bs][D].
    Returns (o1, o2 or None, lse) with o_f [B][Hq][D] and lse [F][B][Hq] (natural log).
    ``batches`` restricts the work to some sequences (other rows stay NaN). ``dtype`` is
    the working precision (float64; float32 evaluates the same definition in single).
    """
    flows = _queries(q1, q2_raw, a, a_head_stride, dtype)
    F = len(flows)
    B, Hq, D = flows[0].shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if softmax_scale is None or softmax_scale <= 0 else float(softmax_scale)
    out = [np.full((B, Hq, D), np.nan) for _ in range(F)]
    lse = np.full((F, B, Hq), np.nan)
    weights = {}
    ctx = np.asarray(context_lens)
    for b in (range(B) if batches is None else batches):
        n = int(ctx[b])
        if n == 0:
            for f in range(F):
                out[f][b] = 0.0
            lse[:, b] = -np.inf
            continue
        K = widen(gather_kv(k_pool, block_table, b, n)).astype(dtype)
        V = widen(gather_kv(v_pool, block_table, b, n)).astype(dtype)
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            Q = np.concatenate([fl[b, heads] for fl in flows], axis=0)      # [F*G][D]
            S = dtype(scale) * (Q @ K[g].T)                                 # [F*G][n]
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1, keepdims=True)
            W = E / l
            O = W @ V[g]
            for f in range(F):
                out[f][b, heads] = O[f * G:(f + 1) * G]
                lse[f, b, heads] = (m + np.log(l))[f * G:(f + 1) * G, 0]
            if return_weights:
                weights[(b, g)] = W
    res = (out[0], out[1] if F == 2 else None, lse)
    return res + (weights,) if return_weights else res


def brute_force(q1, q2_raw, a, a_head_stride, k_pool, v_pool, block_table, context_lens,
                softmax_scale=None):
    """The same definition as scalar Python loops, for tiny shapes only."""
    q1 = widen(q1)
    B, Hq, D = q1.shape
    Hkv, bs = k_pool.shape[1], k_pool.shape[2]
    G = Hq // Hkv
    kp, vp = widen(k_pool), widen(v_pool)
    q2 = widen(q2_raw) if q2_raw is not None else None
    av = widen(a) if a is not None else None
    scale = 1.0 / math.sqrt(D) if softmax_scale is None or softmax_scale <= 0 else float(softmax_scale)
    F = 1 if q2 is None else 2
    o = np.zeros((F, B, Hq, D))
    lse = np.zeros((F, B, Hq))
    for b in range(B):
        n = int(context_lens[b])
        for h in range(Hq):
            g = h // G
            for f in range(F):
                q = [0.0] * D
                for d in range(D):
                    if f == 0:
                        q[d] = q1[b, h, d]
                    else:
                        coup = 0.0
                        if av is not None:
                            coup = (av[d] if a_head_stride == 0 else av[h, d]) * q1[b, h, d]
                        q[d] = q2[b, h, d] + coup
                if n == 0:
                    lse[f, b, h] = -math.inf
                    continue
                rows = []
                for p in range(n):
                    if block_table is None:
                        blk, slot = b, p
                    else:
                        blk, slot = int(block_table[b][p // bs]), p % bs
                    s = 0.0
                    for d in range(D):
                        s += q[d] * kp[blk, g, slot, d]
                    rows.append((scale * s, blk, slot))
                mx = max(r[0] for r in rows)
                den = 0.0
                acc = [0.0] * D
                for s, blk, slot in rows:
                    e = math.exp(s - mx)
                    den += e
                    for d in range(D):
                        acc[d] += e * vp[blk, g, slot, d]
                for d in range(D):
                    o[f, b, h, d] = acc[d] / den
                lse[f, b, h] = mx + math.log(den)
    return o, lse
