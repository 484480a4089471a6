"""Pins for the oracle's multi-layer decode step (CPU only)."""
import numpy as np

import dfx_inputs as gen
from oracle.layer import dual_flow_layer
from oracle.numerics import widen
from oracle.step import dual_flow_step, embed

KW = dict(vocab=50, batch=3, context=12, hidden=64, num_q_heads=4, num_kv_heads=2, head_dim=16,
          intermediate=96, w_std=0.1)


def test_embed_is_the_one_hot_product():
    c = gen.step_case(71, 1, **KW)
    onehot = np.eye(KW["vocab"])[c.tokens]
    x = embed(c.tokens, c.embed_primary, c.embed_aux)
    assert np.array_equal(x[0], onehot @ widen(c.embed_primary))
    assert np.array_equal(x[1], onehot @ widen(c.embed_aux))


def test_step_composes_layers_and_threads_each_cache():
    c = gen.step_case(72, 2, **KW)
    ctx = c.layers[0].cache.context_lens
    got, pools = dual_flow_step(c.tokens, c.embed_primary, c.embed_aux, c.layers, ctx)
    x = np.stack([widen(c.embed_primary)[c.tokens], widen(c.embed_aux)[c.tokens]])
    for L, (kp, vp) in zip(c.layers, pools):
        kv = L.cache
        x, wk, wv, _ = dual_flow_layer(x, L.g_attn, L.g_mlp, L.w_qkv, L.w_o, L.w_gate_up, L.w_down, L.a, L.b,
                                       L.c, L.eps, kv.k_pool, kv.v_pool, kv.block_table, ctx,
                                       L.num_q_heads, L.num_kv_heads, L.head_dim)
        assert np.array_equal(kp, wk) and np.array_equal(vp, wv)
    assert np.array_equal(got, x)


def test_shared_table_and_no_coupling_make_the_flows_identical():
    c = gen.step_case(73, 2, **KW)
    ctx = c.layers[0].cache.context_lens
    x, _ = dual_flow_step(c.tokens, c.embed_primary, c.embed_primary, c.layers, ctx, couple=False)
    assert np.array_equal(x[0], x[1])
    y, _ = dual_flow_step(c.tokens, c.embed_primary, c.embed_aux, c.layers, ctx, couple=False)
    assert not np.array_equal(y[0], y[1])


def test_primary_and_caches_blind_to_the_aux_table():
    c = gen.step_case(74, 2, **KW)
    ctx = c.layers[0].cache.context_lens
    x1, p1 = dual_flow_step(c.tokens, c.embed_primary, c.embed_aux, c.layers, ctx)
    other = c.embed_aux[::-1].copy()
    x2, p2 = dual_flow_step(c.tokens, c.embed_primary, other, c.layers, ctx)
    x0, p0 = dual_flow_step(c.tokens, c.embed_primary, None, c.layers, ctx)
    assert np.array_equal(x1[0], x2[0]) and np.array_equal(x1[0], x0[0])
    for (a, b), (c1, d1), (e, f) in zip(p1, p2, p0):
        assert np.array_equal(a, c1) and np.array_equal(b, d1) and np.array_equal(a, e) and np.array_equal(b, f)
    assert not np.array_equal(x1[1], x2[1])
