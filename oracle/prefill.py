"""Prefill of a prompt by the primary flow alone, and where the auxiliary flow starts
(oracle, fp64).

What is computed (Sintesi Tecnica: Dual-Flow Transformers, "Architettura Core" and "Costi di
Inferenza vs. Addestramento"; the same in the Japanese summary's description of the method):
during prefill the auxiliary flow is skipped entirely and the primary is an ordinary causal
Transformer that writes the persistent cache; the auxiliary flow starts at the last prompt
position. Reading: a prompt of n tokens is a prefill of tokens 0 .. n-2 by the primary, then
a decode step with both flows at position n-1 (which appends that token's key and value).

prefill_attention: query t of sequence b attends to positions [0, start_b + t], which is the
decode attention of that one query with context start_b + t + 1 (composition of the pinned
decode attention). prefill_dual_attention: the same with both flows' queries at every
position, the forward of the attention at training time, when both flows run over the whole
sequence. prefill_layer: the decode layer's steps for the primary, applied to the T
rows of every sequence at once, with the same bf16 rounding points (normed rows, appended
keys and values, attention rows, normed rows, MLP intermediate).
"""
import numpy as np

from .attention import decode_attention
from .cache import kv_append
from .linear import grouped_linear, rmsnorm, swiglu_couple
from .numerics import bf16_bits, widen


def prefill_attention(q, k_pool, v_pool, block_table, start_pos, batches=None, dtype=np.float64):
    """q: [B][T][Hq][D]; the chunk's keys and values are already in the pools at positions
    start_pos[b] + t. Returns o [B][T][Hq][D] and lse [B][T][Hq] (natural log)."""
    q = np.asarray(q)
    B, T, Hq, D = q.shape
    start = np.asarray(start_pos, np.int64)
    o = np.full((B, T, Hq, D), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    for t in range(T):
        o1, _, l = decode_attention(q[:, t], None, None, 0, k_pool, v_pool, block_table, start + t + 1,
                                    batches=batches, dtype=dtype)
        o[:, t], lse[:, t] = o1, l[0]
    return o, lse


def prefill_dual_attention(q1, q2_raw, a, a_head_stride, k_pool, v_pool, block_table, start_pos, batches=None,
                           dtype=np.float64):
    """Both flows at every new position: the training-time forward of the attention (the
    summary's cost section: training runs both flows over the whole sequence). Query t of
    either flow attends to positions [0, start_b + t] of the primary's cache, which is the
    pinned decode attention of that position's two queries (Q2 = q2_raw + a (.) Q1) with
    context start_b + t + 1. q1, q2_raw: [B][T][Hq][D]; a: [D] (stride 0) or [Hq][D] (stride D)
    or None. Returns o1, o2 [B][T][Hq][D] and lse [2][B][T][Hq] (natural log)."""
    q1, q2_raw = np.asarray(q1), np.asarray(q2_raw)
    B, T, Hq, D = q1.shape
    start = np.asarray(start_pos, np.int64)
    o1 = np.full((B, T, Hq, D), np.nan)
    o2 = np.full((B, T, Hq, D), np.nan)
    lse = np.full((2, B, T, Hq), np.nan)
    for t in range(T):
        r1, r2, l = decode_attention(q1[:, t], q2_raw[:, t], a, a_head_stride, k_pool, v_pool, block_table,
                                     start + t + 1, batches=batches, dtype=dtype)
        o1[:, t], o2[:, t], lse[:, :, t] = r1, r2, l
    return o1, o2, lse


def prefill_layer(x, g_attn, g_mlp, w_qkv, w_o, w_gate_up, w_down, eps, k_pool, v_pool, block_table,
                  start_pos, num_q_heads, num_kv_heads, head_dim, dtype=np.float64):
    """x: float [B][T][hidden] primary rows of positions start_pos[b] + t. Returns (x_out fp64
    [B][T][hidden], k_pool', v_pool', dict of intermediates)."""
    x = np.asarray(x, np.float64)
    B, T, H = x.shape
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    rows = x.reshape(1, B * T, H)
    h1 = rmsnorm(rows, g_attn, eps, dtype)                                 # R1
    qkv = grouped_linear(h1, w_qkv, dtype=dtype)[0].reshape(B, T, -1)
    q = qkv[..., : Hq * D].reshape(B, T, Hq, D)
    k_new = bf16_bits(qkv[..., Hq * D: (Hq + Hkv) * D])                   # R2
    v_new = bf16_bits(qkv[..., (Hq + Hkv) * D:])
    start = np.asarray(start_pos, np.int64)
    kp, vp = k_pool, v_pool
    for t in range(T):
        kp, vp = kv_append(kp, vp, block_table, start + t, k_new[:, t], v_new[:, t])
    o, _ = prefill_attention(q, kp, vp, block_table, start, dtype=dtype)
    o = o.reshape(1, B * T, Hq * D)
    x1 = grouped_linear(o, w_o, residual=rows, dtype=dtype)                # R3 inside
    h2 = rmsnorm(x1, g_mlp, eps, dtype)                                    # R4
    gu = grouped_linear(h2, w_gate_up, dtype=dtype)
    inter = swiglu_couple(gu, None, dtype)                                 # R5
    x2 = grouped_linear(inter, w_down, residual=x1, dtype=dtype)
    mid = dict(h1=h1, qkv=qkv, o=o, x1=x1, h2=h2, inter=inter)
    return x2[0].reshape(B, T, H), kp, vp, mid


def prefill_step(tokens, table_primary, layers, start_pos, dtype=np.float64):
    """tokens: int [B][T] at positions start_pos[b] + t; layers: LayerCase-like objects with
    their caches. The primary's embeddings, then prefill_layer layer by layer. Returns (x_out
    [B][T][hidden], [(k_pool', v_pool')])."""
    x = widen(table_primary)[np.asarray(tokens)]
    pools = []
    for L in layers:
        kv = L.cache
        x, kp, vp, _ = prefill_layer(x, L.g_attn, L.g_mlp, L.w_qkv, L.w_o, L.w_gate_up, L.w_down, L.eps,
                                     kv.k_pool, kv.v_pool, kv.block_table, start_pos, L.num_q_heads,
                                     L.num_kv_heads, L.head_dim, dtype=dtype)
        pools.append((kp, vp))
    return x, pools


def prefill_layer_rows(x, g_attn, g_mlp, w_qkv, w_o, w_gate_up, w_down, eps, num_q_heads, num_kv_heads,
                       head_dim, samples, dtype=np.float64):
    """prefill_layer's output rows at the (sequence, position) pairs ``samples`` of a chunk that
    starts at position 0 (nothing cached before it), for chunks too long to run whole: the same
    steps and rounding points, with every row normed and projected to Q/K/V (the chunk's keys
    and values), and attention, W_o with the residual, the MLP norm, gate/up with SwiGLU and
    W_down run for the sampled rows only. The chunk's keys and values are held as a cache of one
    block per sequence. Returns (x_out [len(samples)][hidden] fp64, k, v) with k, v bf16 bits
    [B][T][Hkv][D]."""
    x = np.asarray(x, np.float64)
    B, T, H = x.shape
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    rows = x.reshape(1, B * T, H)
    qkv = grouped_linear(rmsnorm(rows, g_attn, eps, dtype), w_qkv, dtype=dtype)[0].reshape(B, T, -1)
    k = bf16_bits(qkv[..., Hq * D: (Hq + Hkv) * D]).reshape(B, T, Hkv, D)
    v = bf16_bits(qkv[..., (Hq + Hkv) * D:]).reshape(B, T, Hkv, D)
    k_pool = np.ascontiguousarray(k.transpose(0, 2, 1, 3))  # block b = sequence b
    v_pool = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
    o = np.empty((1, len(samples), Hq * D))
    for i, (b, t) in enumerate(samples):
        o1, _, _ = decode_attention(qkv[b, t, : Hq * D].reshape(1, Hq, D), None, None, 0, k_pool, v_pool,
                                    np.array([[b]], np.int32), np.array([t + 1], np.int32), dtype=dtype)
        o[0, i] = o1.reshape(-1)
    res = rows[:, [b * T + t for b, t in samples]]
    x1 = grouped_linear(o, w_o, residual=res, dtype=dtype)
    inter = swiglu_couple(grouped_linear(rmsnorm(x1, g_mlp, eps, dtype), w_gate_up, dtype=dtype), None, dtype)
    x2 = grouped_linear(inter, w_down, residual=x1, dtype=dtype)
    return x2[0], k, v
