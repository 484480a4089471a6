"""Pins for the oracle's primary-only prefill and the auxiliary flow's start (CPU only).

Checked against torch's causal scaled-dot-product attention, against the token-by-token
recurrence of the separately pinned decode layer (prefilling T tokens at once must equal T
single-token decode steps of the primary), chunking invariance, and the property that makes
skipping the auxiliary during prefill lossless: the auxiliary keeps no state of its own, so
its row at the last prompt position is the same whether or not it ran at earlier positions."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
from oracle.layer import dual_flow_layer
from oracle.numerics import widen
from oracle.prefill import (prefill_attention, prefill_dual_attention, prefill_layer, prefill_layer_rows,
                            prefill_step)
from oracle.step import dual_flow_step

SMALL = dict(hidden=64, num_q_heads=4, num_kv_heads=2, head_dim=32, intermediate=64, w_std=0.1)


def test_prefill_attention_matches_torch_causal_sdpa():
    B, T, Hq, Hkv, D, P = 2, 9, 4, 2, 32, 5            # 5 tokens already cached, 9 new ones
    c = gen.attention_case(31, B, Hq, Hkv, D, np.full(B, P + T, np.int32), "f32", paged=True, block_size=4)
    q = np.random.default_rng(1).standard_normal((B, T, Hq, D))
    o, lse = prefill_attention(q, c.k_pool, c.v_pool, c.block_table, np.full(B, P))
    for b in range(B):
        blocks = c.block_table[b, : -(-(P + T) // 4)]
        K = torch.from_numpy(widen(c.k_pool[blocks]).transpose(1, 0, 2, 3).reshape(Hkv, -1, D)[:, : P + T])
        V = torch.from_numpy(widen(c.v_pool[blocks]).transpose(1, 0, 2, 3).reshape(Hkv, -1, D)[:, : P + T])
        K, V = K.repeat_interleave(Hq // Hkv, 0), V.repeat_interleave(Hq // Hkv, 0)
        Q = torch.from_numpy(q[b].transpose(1, 0, 2))                   # [Hq][T][D]
        mask = torch.arange(P + T)[None, :] <= (P + torch.arange(T))[:, None]
        want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask).numpy()
        assert np.allclose(o[b].transpose(1, 0, 2), want, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_dual_prefill_attention_matches_two_causal_sdpa():
    """Both flows at every position against torch's causal SDPA per flow, the auxiliary's query
    materialised as q2_raw + a * q1 (per-head a), over the primary's keys and values."""
    B, T, Hq, Hkv, D, P = 2, 7, 4, 2, 32, 3
    c = gen.attention_case(33, B, Hq, Hkv, D, np.full(B, P + T, np.int32), "f32", paged=True, block_size=4)
    rng = np.random.default_rng(5)
    q1, q2 = rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hq, D))
    a = rng.uniform(-1, 1, (Hq, D))
    o1, o2, lse = prefill_dual_attention(q1, q2, a, D, c.k_pool, c.v_pool, c.block_table, np.full(B, P))
    mask = torch.arange(P + T)[None, :] <= (P + torch.arange(T))[:, None]
    for b in range(B):
        blocks = c.block_table[b, : -(-(P + T) // 4)]
        K = torch.from_numpy(widen(c.k_pool[blocks]).transpose(1, 0, 2, 3).reshape(Hkv, -1, D)[:, : P + T])
        V = torch.from_numpy(widen(c.v_pool[blocks]).transpose(1, 0, 2, 3).reshape(Hkv, -1, D)[:, : P + T])
        K, V = K.repeat_interleave(Hq // Hkv, 0), V.repeat_interleave(Hq // Hkv, 0)
        for q, o in ((q1[b], o1[b]), (q2[b] + a[None] * q1[b], o2[b])):
            Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))          # [Hq][T][D]
            want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask).numpy()
            assert np.allclose(o.transpose(1, 0, 2), want, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_dual_prefill_attention_flow_properties():
    """Adding the auxiliary leaves the primary's rows exactly as the primary-only attention's;
    Q2 = Q1 (q2_raw = q1, a = 0) gives the auxiliary exactly the primary's rows."""
    B, T, Hq, Hkv, D, P = 2, 5, 4, 1, 32, 6
    c = gen.attention_case(34, B, Hq, Hkv, D, np.full(B, P + T, np.int32), "f32", paged=True, block_size=4)
    rng = np.random.default_rng(6)
    q1, q2 = rng.standard_normal((B, T, Hq, D)), rng.standard_normal((B, T, Hq, D))
    st = np.full(B, P)
    o1, _, lse = prefill_dual_attention(q1, q2, rng.uniform(-1, 1, D), 0, c.k_pool, c.v_pool, c.block_table, st)
    p1, pl = prefill_attention(q1, c.k_pool, c.v_pool, c.block_table, st)
    assert np.array_equal(o1, p1) and np.array_equal(lse[0], pl)
    s1, s2, sl = prefill_dual_attention(q1, q1, np.zeros(D), 0, c.k_pool, c.v_pool, c.block_table, st)
    assert np.array_equal(s1, s2) and np.array_equal(sl[0], sl[1])


def prefill_case(seed, B=2, start=3, T=6):
    return gen.layer_case(seed, batch=B, context=start + 1, capacity=start + T + 1, block_size=4, **SMALL)


def test_prefill_layer_equals_token_by_token_decode():
    start, T = 3, 6
    c = prefill_case(41, start=start, T=T)
    xs = np.random.default_rng(2).standard_normal((2, T, c.hidden)).astype(np.float32)
    kv = c.cache
    st = np.full(2, start)
    got, kp, vp, _ = prefill_layer(xs, c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down, c.eps,
                                   kv.k_pool, kv.v_pool, kv.block_table, st, c.num_q_heads, c.num_kv_heads,
                                   c.head_dim)
    kq, vq = kv.k_pool, kv.v_pool
    for t in range(T):
        y, kq, vq, _ = dual_flow_layer(xs[None, :, t], c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down,
                                       None, None, None, c.eps, kq, vq, kv.block_table, st + t,
                                       c.num_q_heads, c.num_kv_heads, c.head_dim)
        assert np.allclose(got[:, t], y[0], rtol=0, atol=1e-9)
    assert np.array_equal(kp, kq) and np.array_equal(vp, vq)


def test_sampled_prefill_rows_equal_the_whole_layer():
    """The sampled-row composition (for chunks too long to run whole) reproduces prefill_layer
    from position 0 at every sampled row, and its keys and values are the ones prefill_layer
    appends, gathered through the block table."""
    T = 11
    c = prefill_case(44, start=0, T=T)
    xs = np.random.default_rng(5).standard_normal((2, T, c.hidden)).astype(np.float32)
    kv = c.cache
    whole, kp, vp, _ = prefill_layer(xs, c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down, c.eps,
                                     kv.k_pool, kv.v_pool, kv.block_table, np.zeros(2), c.num_q_heads,
                                     c.num_kv_heads, c.head_dim)
    samples = [(0, 0), (0, 5), (1, 10), (1, 3), (0, 10)]
    rows, k, v = prefill_layer_rows(xs, c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down, c.eps,
                                    c.num_q_heads, c.num_kv_heads, c.head_dim, samples)
    for i, (b, t) in enumerate(samples):
        assert np.allclose(rows[i], whole[b, t], rtol=0, atol=1e-12)
    bs = kv.k_pool.shape[2]
    for b in range(2):
        for t in range(T):
            blk = kv.block_table[b, t // bs]
            assert np.array_equal(k[b, t], kp[blk, :, t % bs]) and np.array_equal(v[b, t], vp[blk, :, t % bs])


def test_chunked_prefill_equals_one_chunk():
    c = prefill_case(42, start=2, T=7)
    xs = np.random.default_rng(3).standard_normal((2, 7, c.hidden)).astype(np.float32)
    kv = c.cache
    args = (c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down, c.eps)
    heads = (c.num_q_heads, c.num_kv_heads, c.head_dim)
    whole, kw, vw, _ = prefill_layer(xs, *args, kv.k_pool, kv.v_pool, kv.block_table, np.full(2, 2), *heads)
    a, ka, va, _ = prefill_layer(xs[:, :3], *args, kv.k_pool, kv.v_pool, kv.block_table, np.full(2, 2), *heads)
    b, kb, vb, _ = prefill_layer(xs[:, 3:], *args, ka, va, kv.block_table, np.full(2, 5), *heads)
    assert np.allclose(np.concatenate([a, b], 1), whole, rtol=0, atol=1e-9)
    assert np.array_equal(kb, kw) and np.array_equal(vb, vw)


def test_aux_starts_at_the_last_prompt_position_without_loss():
    """Prompt of n tokens: prefill of n - 1 tokens by the primary, then one dual step at
    position n - 1. Running both flows at every position instead gives the same rows at the
    last position and the same caches: the auxiliary writes no cache and carries no state."""
    n, B, start = 5, 2, 0
    layers = [prefill_case(50 + l, B=B, start=start, T=n) for l in range(2)]
    rng = np.random.default_rng(4)
    vocab = 11
    e1 = gen.f32_to_bf16_bits(rng.standard_normal((vocab, SMALL["hidden"])).astype(np.float32))
    e2 = gen.f32_to_bf16_bits(rng.standard_normal((vocab, SMALL["hidden"])).astype(np.float32))
    tokens = rng.integers(0, vocab, (B, n))
    # the method: primary-only prefill, then the auxiliary starts
    _, pools = prefill_step(tokens[:, : n - 1], e1, layers, np.full(B, start))
    for L, (kp, vp) in zip(layers, pools):
        L.cache.k_pool, L.cache.v_pool = kp, vp
    x_last, pools_last = dual_flow_step(tokens[:, n - 1], e1, e2, layers, np.full(B, start + n - 1))
    # both flows at every position
    fresh = [prefill_case(50 + l, B=B, start=start, T=n) for l in range(2)]
    for t in range(n):
        x_all, pools_all = dual_flow_step(tokens[:, t], e1, e2, fresh, np.full(B, start + t))
        for L, (kp, vp) in zip(fresh, pools_all):
            L.cache.k_pool, L.cache.v_pool = kp, vp
    assert np.allclose(x_all, x_last, rtol=0, atol=1e-9)
    for (ka, va), (kb, vb) in zip(pools_all, pools_last):
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
