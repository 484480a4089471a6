"""Pins for the oracle's dual-flow decode layer (CPU only).

The primary flow of the layer is checked against a textbook pre-norm decoder
layer written with torch.nn.functional (rms_norm, linear, SDPA with grouped
KV heads, silu) in fp64, rounding to bf16 at the same five points; its cache
comes from the input generator's logical rows plus the new token, not from the
oracle's pool and table. The auxiliary flow is pinned by identities.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import dfx_inputs as gen
from oracle.layer import dual_flow_layer
from oracle.numerics import round_bf16, widen

SMALL = dict(batch=2, context=20, hidden=64, num_q_heads=4, num_kv_heads=2, head_dim=16,
             intermediate=96, w_std=0.1)


def run(c, x=None, a="c", b="c", cc="c", flows=2):
    x = c.x if x is None else x
    a = c.a if isinstance(a, str) else a
    b = c.b if isinstance(b, str) else b
    cc = c.c if isinstance(cc, str) else cc
    kv = c.cache
    return dual_flow_layer(x[:flows], c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down,
                           a, b, cc, c.eps, kv.k_pool, kv.v_pool, kv.block_table, kv.context_lens,
                           c.num_q_heads, c.num_kv_heads, c.head_dim)


def T(a):
    return torch.from_numpy(widen(a))


def R(t):
    return torch.from_numpy(round_bf16(t.numpy()))


def textbook_primary(c):
    B, H, Hq, Hkv, D, I = c.batch, c.hidden, c.num_q_heads, c.num_kv_heads, c.head_dim, c.intermediate
    x = torch.from_numpy(c.x[0].astype(np.float64))
    h = R(Fn.rms_norm(x, (H,), weight=T(c.g_attn), eps=c.eps))
    qkv = Fn.linear(h, T(c.w_qkv))
    q, k, v = qkv.split([Hq * D, Hkv * D, Hkv * D], dim=-1)
    k, v = R(k), R(v)
    out = []
    for bi in range(B):
        n = int(c.cache.context_lens[bi])
        ks, vs = [], []
        for g in range(Hkv):
            kg = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(gen._normal(c.seed, gen.TID_K, (bi, g), (n, D))))
            vg = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(gen._normal(c.seed, gen.TID_V, (bi, g), (n, D))))
            ks.append(torch.cat([torch.from_numpy(kg.astype(np.float64)), k[bi, g * D:(g + 1) * D][None]]))
            vs.append(torch.cat([torch.from_numpy(vg.astype(np.float64)), v[bi, g * D:(g + 1) * D][None]]))
        K, V = torch.stack(ks)[None], torch.stack(vs)[None]          # [1][Hkv][n+1][D]
        Q = q[bi].view(1, Hq, 1, D)
        out.append(Fn.scaled_dot_product_attention(Q, K, V, enable_gqa=True).reshape(Hq * D))
    o = torch.stack(out)
    x1 = x + Fn.linear(R(o), T(c.w_o))
    h2 = R(Fn.rms_norm(x1, (H,), weight=T(c.g_mlp), eps=c.eps))
    gate, up = Fn.linear(h2, T(c.w_gate_up)).split([I, I], dim=-1)
    inter = R(Fn.silu(gate) * up)
    return (x1 + Fn.linear(inter, T(c.w_down))).numpy()


@pytest.fixture(scope="module")
def case():
    return gen.layer_case(77, **SMALL)


def test_primary_is_a_textbook_decoder_layer(case):
    y, _, _, _ = run(case)
    assert np.max(np.abs(y[0] - textbook_primary(case))) < 1e-12


def test_primary_ignores_the_auxiliary_flow(case):
    y2, kp2, vp2, _ = run(case, flows=2)
    y1, kp1, vp1, _ = run(case, flows=1)
    assert np.array_equal(y2[0], y1[0])
    assert np.array_equal(kp1, kp2) and np.array_equal(vp1, vp2)       # aux writes no cache
    other = case.x.copy()
    other[1] = -3 * other[1] + 1
    y3, kp3, _, _ = run(case, x=other, a=np.full(case.head_dim, 0.5, np.float32))
    assert np.array_equal(y3[0], y2[0]) and np.array_equal(kp3, kp2)


def test_aux_equals_primary_without_coupling(case):
    x = np.stack([case.x[0], case.x[0]])
    y, _, _, _ = run(case, x=x, a=None, b=None, cc=None)
    assert np.array_equal(y[0], y[1])
    z = np.zeros
    y0, _, _, _ = run(case, x=x, a=z(case.head_dim, np.float32), b=z(case.intermediate, np.float32),
                      cc=z(case.hidden, np.float32))
    assert np.array_equal(y0[0], y0[1]) and np.array_equal(y0[0], y[0])


def test_b_and_c_coupling_identities(case):
    # equal rows, a = 0: b = -1 zeroes the aux MLP intermediate, so the aux MLP output is
    # c * m_prim alone; with c = -1 the two flows' outputs average to the post-attention row
    x = np.stack([case.x[0], case.x[0]])
    H, I = case.hidden, case.intermediate
    y, _, _, mid = run(case, x=x, a=np.zeros(case.head_dim, np.float32),
                       b=np.full(I, -1.0, np.float32), cc=np.full(H, -1.0, np.float32))
    assert np.all(mid["inter"][1] == 0)
    assert np.max(np.abs((y[0] + y[1]) / 2 - mid["x1"][0])) < 1e-12
    y, _, _, mid = run(case, x=x, a=np.zeros(case.head_dim, np.float32),
                       b=np.full(I, -1.0, np.float32), cc=np.zeros(H, np.float32))
    assert np.array_equal(y[1], mid["x1"][1])


def test_cache_diff_is_exactly_the_primary_rows(case):
    _, kp, vp, mid = run(case)
    kv = case.cache
    Hq, Hkv, D = case.num_q_heads, case.num_kv_heads, case.head_dim
    changed = np.argwhere(np.any(kp != kv.k_pool, axis=-1))
    assert len(changed) == case.batch * Hkv
    for b in range(case.batch):
        p = int(kv.context_lens[b])
        blk, slot = int(kv.block_table[b][p // 16]), p % 16
        k_row = mid["qkv"][0, b, Hq * D:(Hq + Hkv) * D].reshape(Hkv, D)
        v_row = mid["qkv"][0, b, (Hq + Hkv) * D:].reshape(Hkv, D)
        assert np.array_equal(widen(kp[blk, :, slot]), round_bf16(k_row))
        assert np.array_equal(widen(vp[blk, :, slot]), round_bf16(v_row))
