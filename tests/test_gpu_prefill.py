"""GPU parity of the primary-only prefill (dfx_prefill_attn, dfx_prefill_layer, dfx_prefill_step),
of the auxiliary flow's start at the last prompt position, and of the causal attention with
both flows at every position (dfx_prefill_dual_attn, the training-time forward).

Tolerances: the causal attention outputs against the oracle at max-abs 2e-3 (bf16 cache) and,
tighter, 5e-5 (Q and P are split into three bf16 terms, every fp32 bit); the layer and step
outputs within twice the distance of an ensemble of fp32 evaluations of the oracle
(tests/twins.py), as the decode layer's; the appended keys and values equal bit for bit but for
rare rounding decisions one bf16 step apart (fp32 against fp64 projections); chunked prefill
bit-identical to one chunk."""
import copy

import numpy as np
import pytest
import torch

import dfx_inputs as gen
import dual_flow_shared_amd as dfx
from gpu_util import cache_of, dev, host_bits
from oracle.prefill import (prefill_attention, prefill_dual_attention, prefill_layer, prefill_layer_rows,
                            prefill_step)
from oracle.linear import rmsnorm
from oracle.numerics import widen
from oracle.step import dual_flow_step
from twins import assert_twin_close, twin_errors
from gpu_util import bf16_decisions_agree, unpack_rows
from oracle.attention import decode_attention, gather_kv
from oracle.linear import grouped_linear, swiglu_couple
from test_gpu_layer import U, attention_row_bound, gamma, norm_bound

pytestmark = pytest.mark.gpu


def prefill_twins(c, x, st, want):
    """fp32 ensemble distances of prefill_layer on the chunk x (tests/twins.py)."""
    return twin_errors(lambda d, ph: prefill_layer(x[..., ph], d.g_attn, d.g_mlp, d.w_qkv, d.w_o, d.w_gate_up,
                                                   d.w_down, d.eps, d.cache.k_pool, d.cache.v_pool, d.cache.block_table,
                                                   st, d.num_q_heads, d.num_kv_heads, d.head_dim, dtype=np.float32)[0],
                       c, want)


@pytest.mark.parametrize("paged,D,Hq,Hkv,T,starts", [
    (True, 128, 8, 2, 37, [0, 21]),        # ragged tail tile, different start per sequence
    (True, 128, 32, 8, 16, [5, 0]),
    (False, 64, 4, 4, 50, [3, 7]),         # contiguous cache, head_dim 64, no grouping
    (True, 128, 8, 1, 1, [40, 0]),         # one new position (a decode-shaped chunk)
    (True, 128, 8, 4, 33, [2, 17]),        # two heads per KV head: the per-wave K/V kernel
])
def test_prefill_attention(paged, D, Hq, Hkv, T, starts):
    B = len(starts)
    st = np.array(starts, np.int32)
    ctx = st + T
    c = gen.attention_case(600 + T, B, Hq, Hkv, D, ctx, "bf16", paged=paged, block_size=16,
                           capacity=int(ctx.max()) + 16)
    q = np.random.default_rng(T).standard_normal((B, T, Hq, D)).astype(np.float32)
    cache = cache_of(c)
    o, lse = dfx.prefill_attn(dev(q), cache, dev(st), int(ctx.max()) + 16, want_lse=True)
    torch.cuda.synchronize()
    want, wl = prefill_attention(q, c.k_pool, c.v_pool, c.block_table, st)
    err = np.abs(o.cpu().numpy() - want).max()
    assert err < 2e-3 and err < 5e-5, err
    assert np.abs(lse.cpu().numpy() - wl).max() < 1e-4


@pytest.mark.parametrize("paged,D,Hq,Hkv,T,starts,per_head", [
    (True, 128, 8, 2, 37, [0, 21], False),   # K/V tiles shared through LDS, ragged tail tile
    (False, 128, 32, 8, 16, [5, 0], True),   # the same, contiguous cache, per-head a
    (True, 64, 4, 4, 50, [3, 7], False),     # per-wave kernel, head_dim 64
    (True, 128, 8, 4, 33, [2, 17], True),    # per-wave kernel, head_dim 128
    (True, 128, 8, 1, 1, [40, 0], False),    # one position
])
def test_prefill_dual_attention(paged, D, Hq, Hkv, T, starts, per_head):
    """Both flows at every position against the oracle; the primary's rows bit-identical to
    the primary-only call's; Q2 = Q1 gives the auxiliary exactly the primary's rows."""
    B = len(starts)
    st = np.array(starts, np.int32)
    ctx = st + T
    c = gen.attention_case(650 + T, B, Hq, Hkv, D, ctx, "bf16", paged=paged, block_size=16,
                           capacity=int(ctx.max()) + 16)
    rng = np.random.default_rng(T + D)
    q1 = rng.standard_normal((B, T, Hq, D)).astype(np.float32)
    q2 = rng.standard_normal((B, T, Hq, D)).astype(np.float32)
    a = rng.uniform(-1, 1, (Hq, D) if per_head else D).astype(np.float32)
    cache = cache_of(c)
    mc = int(ctx.max()) + 16
    q1t, stt = dev(q1), dev(st)
    o1, o2, lse = dfx.prefill_dual_attn(q1t, dev(q2), dev(a), cache, stt, mc, want_lse=True)
    p1 = dfx.prefill_attn(q1t, cache, stt, mc)
    s1, s2 = dfx.prefill_dual_attn(q1t, q1t, None, cache, stt, mc)
    torch.cuda.synchronize()
    w1, w2, wl = prefill_dual_attention(q1, q2, a, D if per_head else 0, c.k_pool, c.v_pool, c.block_table, st)
    for got, want in ((o1, w1), (o2, w2)):
        err = np.abs(got.cpu().numpy() - want).max()
        assert err < 2e-3 and err < 5e-5, err
    assert np.abs(lse.cpu().numpy() - wl).max() < 1e-4
    assert torch.equal(o1, p1)
    assert torch.equal(s1, s2) and torch.equal(s1, p1)


def test_prefill_attention_full_size_sampled_positions():
    """The prefill benchmark's attention calls (2 sequences x 2048 positions from position 0,
    32/8 heads x 128, paged bf16 cache of 16-token blocks in a permuted pool): every head of
    both sequences at sampled positions against the oracle's one-position chunk starting there,
    for the primary-only call and both flows; the two calls' primary rows bit-identical."""
    B, T, Hq, Hkv, D = 2, 2048, 32, 8, 128
    st = np.zeros(B, np.int32)
    c = gen.attention_case(690, B, Hq, Hkv, D, np.full(B, T, np.int32), "bf16", paged=True, block_size=16,
                           capacity=T + 16)
    rng = np.random.default_rng(12)
    q1 = rng.standard_normal((B, T, Hq, D)).astype(np.float32)
    q2 = rng.standard_normal((B, T, Hq, D)).astype(np.float32)
    a = rng.uniform(-1, 1, D).astype(np.float32)
    cache = cache_of(c)
    q1t, stt = dev(q1), dev(st)
    print(f"prefill attention B={B} T={T}", flush=True)
    p1, pl = dfx.prefill_attn(q1t, cache, stt, T + 16, want_lse=True)
    o1, o2, lse = dfx.prefill_dual_attn(q1t, dev(q2), dev(a), cache, stt, T + 16, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, p1)
    p1, pl, o2, lse = p1.cpu().numpy(), pl.cpu().numpy(), o2.cpu().numpy(), lse.cpu().numpy()
    for t in [0, 1, 15, 16, 31, 32, 1000, T - 2, T - 1] + [int(u) for u in rng.integers(0, T, 5)]:
        w1, wl1 = prefill_attention(q1[:, [t]], c.k_pool, c.v_pool, c.block_table, st + t)
        d1, d2, dl = prefill_dual_attention(q1[:, [t]], q2[:, [t]], a, 0, c.k_pool, c.v_pool, c.block_table, st + t)
        for got, want in ((p1[:, t], w1[:, 0]), (p1[:, t], d1[:, 0]), (o2[:, t], d2[:, 0])):
            err = np.abs(got - want).max()
            assert err < 2e-3 and err < 5e-5, (t, err)
        assert np.abs(pl[:, t] - wl1[:, 0]).max() < 1e-4
        assert np.abs(lse[:, :, t] - dl[:, :, 0]).max() < 1e-4


SMALL = dict(hidden=256, num_q_heads=8, num_kv_heads=2, head_dim=128, intermediate=512, w_std=0.05)


def weights_of(c):
    return dfx.LayerWeights.from_row_major(dev(c.g_attn), dev(c.w_qkv), dev(c.w_o), dev(c.g_mlp), dev(c.w_gate_up),
                                           dev(c.w_down), c.num_q_heads, c.num_kv_heads, c.head_dim, c.eps)


def test_prefill_layer_parity_and_appended_rows():
    B, start, T = 3, 19, 45
    c = gen.layer_case(701, batch=B, context=start + 1, capacity=start + T + 8, **SMALL)
    x = np.random.default_rng(3).standard_normal((B, T, c.hidden)).astype(np.float32)
    cache = cache_of(c.cache)
    st = np.full(B, start, np.int32)
    xt = dev(x)
    dfx.prefill_layer(xt, weights_of(c), cache, dev(st), start + T + 8)
    torch.cuda.synchronize()
    want, kp, vp, _ = prefill_layer(x, c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down, c.eps,
                                    c.cache.k_pool, c.cache.v_pool, c.cache.block_table, st, c.num_q_heads,
                                    c.num_kv_heads, c.head_dim)
    assert_twin_close(xt.cpu().numpy(), want, prefill_twins(c, x, st, want), "prefill layer")
    gk, gv = host_bits(cache.k), host_bits(cache.v)
    # the pool changed exactly at the chunk's slots, and agrees with the oracle's appended rows
    changed = np.any(gk != c.cache.k_pool, axis=(1, 3))
    assert np.array_equal(changed, np.any(kp != c.cache.k_pool, axis=(1, 3)))
    for got, ref in ((gk, kp), (gv, vp)):
        # slots the chunk wrote: equal bits but for rare rounding decisions one bf16 step apart
        # (the GPU and the oracle round fp32 and fp64 projections of slightly different rows)
        rows = changed[:, None, :, None] & np.ones_like(got, bool)
        same = got[rows] == ref[rows]
        assert same.mean() > 0.995
        g = gen.bf16_bits_to_f32(got[rows][~same]).astype(np.float64)
        r = gen.bf16_bits_to_f32(ref[rows][~same]).astype(np.float64)
        _, e = np.frexp(np.maximum(np.abs(g), np.abs(r)))
        assert np.all(np.abs(g - r) <= np.ldexp(1.0, e - 8))


def test_prefill_layer_odd_k_steps():
    """hidden 288 and intermediate 544: every projection's K is an odd number of 32-wide
    k-steps (9, 17, 32 for W_o), and 3 x 50 rows make three 64-row groups with a ragged tail."""
    B, start, T = 3, 4, 50
    c = gen.layer_case(703, batch=B, context=start + 1, capacity=start + T + 8, hidden=288, num_q_heads=8,
                       num_kv_heads=2, head_dim=128, intermediate=544, w_std=0.05)
    x = np.random.default_rng(7).standard_normal((B, T, c.hidden)).astype(np.float32)
    cache = cache_of(c.cache)
    st = np.full(B, start, np.int32)
    xt = dev(x)
    dfx.prefill_layer(xt, weights_of(c), cache, dev(st), start + T + 8)
    torch.cuda.synchronize()
    want, _, _, _ = prefill_layer(x, c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down, c.eps,
                                  c.cache.k_pool, c.cache.v_pool, c.cache.block_table, st, c.num_q_heads,
                                  c.num_kv_heads, c.head_dim)
    assert_twin_close(xt.cpu().numpy(), want, prefill_twins(c, x, st, want), "prefill layer")


def kv_step_bound(x, c):
    """How far each appended key/value element [B][T][Hkv][D] of the device may sit from the
    oracle's: one bf16 step of the value, plus the fp32 accumulation bound of the projection,
    gamma(K) sum_k |h1_k w_k| with gamma(K) = (K/32 + 64) 2^-24 (32-term matrix-core blocks added
    in sequence), plus |w_k| ulp(h1_k) for every normed input element whose unrounded value lies
    within 2^-20 (relative) of a bf16 rounding boundary, which the device's fp32 norm may round
    the other way. Returns the bound without the one-step term."""
    B, T, H = x.shape
    Hq, Hkv, D = c.num_q_heads, c.num_kv_heads, c.head_dim
    rows = np.asarray(x, np.float64).reshape(1, B * T, H)
    h1u = rmsnorm(rows, c.g_attn, c.eps, rounded=False)[0]
    h1 = rmsnorm(rows, c.g_attn, c.eps)[0]
    _, e = np.frexp(h1u)
    half = np.ldexp(1.0, e - 9)                                   # half a bf16 step at h1u
    near = half - np.abs(h1u - h1) <= np.ldexp(np.abs(h1u), -20)  # close to a rounding boundary
    w = np.abs(widen(c.w_qkv)[Hq * D:])                          # K and V rows of W_qkv
    gamma = (H / 32 + 64) * 2.0 ** -24
    bound = gamma * (np.abs(h1) @ w.T) + np.where(near, 2 * half, 0.0) @ w.T
    return bound.reshape(B, T, 2, Hkv, D)


@pytest.mark.parametrize("B,T,shape", [
    # the one-layer workload's shape at the prefill benchmark's chunk: the 256 x 256 projection
    # tile on gate/up, W_o and W_down, the 192 x 256 one on Q/K/V
    (2, 2048, dict(hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128, intermediate=14336, w_std=0.02)),
    # the 256 x 256 tile on every projection, with a ragged last row group (7990 rows) and ragged
    # feature tiles (W_o and W_down 288 features, gate/up 1504; down K = 47 k-steps)
    (2, 3995, dict(hidden=288, num_q_heads=4, num_kv_heads=2, head_dim=64, intermediate=1504, w_std=0.05)),
    # the 192 x 256 tile on W_o and W_down with a ragged last feature tile (5984 = 31 x 192 + 32)
    # and a ragged last row group (3980 rows); gate/up on 256 x 256, Q/K/V on 256 x 128
    (2, 1990, dict(hidden=5984, num_q_heads=8, num_kv_heads=2, head_dim=128, intermediate=1504, w_std=0.02)),
    # hidden 64: Q/K/V's and gate/up's K is 2 k-steps, fewer than the 256 x 256 tile keeps in
    # flight (its prologue re-reads the last one); every projection on the 256 x 256 tile
    (2, 3995, dict(hidden=64, num_q_heads=4, num_kv_heads=1, head_dim=64, intermediate=1504, w_std=0.05)),
])
def test_prefill_layer_long_chunk_sampled_rows(B, T, shape):
    """A long chunk from position 0: sampled output rows against the oracle's composition for
    those rows, and every appended key and value.

    Unlike the short chunks, thousands of the attended keys and values are the chunk's own,
    computed and rounded to bf16 on both sides; the rare ones a bf16 step apart (checked below)
    shift late positions' attention rows, and the later rounding points (h2, the MLP
    intermediate) spread that over the row: the median bar is 4e-3 here (measured 2.6e-3 at
    2048 positions; position 0, which attends to one key, 1e-4)."""
    c = gen.layer_case(705, batch=B, context=1, capacity=T + 8, **shape)
    x = np.random.default_rng(9).standard_normal((B, T, c.hidden)).astype(np.float32)
    cache = cache_of(c.cache)
    xt = dev(x)
    print(f"prefill layer B={B} T={T} hidden={c.hidden}", flush=True)
    dfx.prefill_layer(xt, weights_of(c), cache, dev(np.zeros(B, np.int32)), T + 8)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    samples = [(0, 0), (0, T - 1), (1, 0), (1, T - 2), (1, T - 1)]
    samples += [(int(b), int(t)) for b, t in zip(rng.integers(0, B, 11), rng.integers(0, T, 11))]
    want, k, v = prefill_layer_rows(x, c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down, c.eps,
                                    c.num_q_heads, c.num_kv_heads, c.head_dim, samples)
    got = xt.cpu().numpy()
    errs = twin_errors(lambda d, ph: prefill_layer_rows(x[..., ph], d.g_attn, d.g_mlp, d.w_qkv, d.w_o, d.w_gate_up,
                                                        d.w_down, d.eps, d.num_q_heads, d.num_kv_heads, d.head_dim,
                                                        samples, dtype=np.float32)[0], c, want)
    assert_twin_close(np.stack([got[b, t] for b, t in samples]), want, errs, "prefill layer rows")
    bs, tbl, t = c.cache.k_pool.shape[2], c.cache.block_table, np.arange(T)
    bound = kv_step_bound(x, c)
    for i, (pool, ref) in enumerate(((host_bits(cache.k), k), (host_bits(cache.v), v))):
        g = np.stack([pool[tbl[b, t // bs], :, t % bs] for b in range(B)])  # [B][T][Hkv][D]
        same = g == ref
        assert same.mean() > 0.995
        gd = gen.bf16_bits_to_f32(g[~same]).astype(np.float64)
        rd = gen.bf16_bits_to_f32(ref[~same]).astype(np.float64)
        _, e = np.frexp(np.maximum(np.abs(gd), np.abs(rd)))
        assert np.all(np.abs(gd - rd) <= np.ldexp(1.0, e - 8) + bound[:, :, i][~same])


def test_chunked_prefill_is_bit_identical_to_one_chunk():
    B, start, T, T1 = 2, 6, 40, 17
    c = gen.layer_case(702, batch=B, context=start + 1, capacity=start + T + 8, **SMALL)
    x = np.random.default_rng(4).standard_normal((B, T, c.hidden)).astype(np.float32)
    w = weights_of(c)
    mc = start + T + 8
    one = cache_of(c.cache)
    xa = dev(x)
    dfx.prefill_layer(xa, w, one, dev(np.full(B, start, np.int32)), mc)
    two = cache_of(c.cache)
    xb1, xb2 = dev(x[:, :T1].copy()), dev(x[:, T1:].copy())
    dfx.prefill_layer(xb1, w, two, dev(np.full(B, start, np.int32)), mc)
    dfx.prefill_layer(xb2, w, two, dev(np.full(B, start + T1, np.int32)), mc)
    torch.cuda.synchronize()
    assert np.array_equal(torch.cat([xb1, xb2], 1).cpu().numpy(), xa.cpu().numpy())
    assert np.array_equal(host_bits(one.k), host_bits(two.k)) and np.array_equal(host_bits(one.v), host_bits(two.v))


def test_prefill_then_aux_start_matches_oracle():
    """A prompt of n tokens: the primary prefills n - 1 of them, then the decode step with both
    flows at the last position; against the oracle's composition of the same two steps."""
    B, n, L = 2, 24, 2
    vocab = 50
    layers = [gen.layer_case(710 + l, batch=B, context=1, capacity=n + 8, **SMALL) for l in range(L)]
    rng = np.random.default_rng(5)
    e1 = gen.f32_to_bf16_bits(rng.standard_normal((vocab, SMALL["hidden"])).astype(np.float32))
    e2 = gen.f32_to_bf16_bits(rng.standard_normal((vocab, SMALL["hidden"])).astype(np.float32))
    tokens = rng.integers(0, vocab, (B, n)).astype(np.int32)
    caches = [cache_of(Lc.cache) for Lc in layers]
    ws = [dfx.LayerWeights.from_row_major(dev(Lc.g_attn), dev(Lc.w_qkv), dev(Lc.w_o), dev(Lc.g_mlp),
                                          dev(Lc.w_gate_up), dev(Lc.w_down), Lc.num_q_heads, Lc.num_kv_heads,
                                          Lc.head_dim, Lc.eps, dev(Lc.a), dev(Lc.b), dev(Lc.c)) for Lc in layers]
    zero = dev(np.zeros(B, np.int32))
    xp = dfx.prefill_step(dev(tokens[:, : n - 1].copy()), dev(e1), ws, caches, zero, n + 8)
    ctx = dev(np.full(B, n, np.int32))
    x_last = dfx.dual_flow_decode_step(dev(tokens[:, n - 1].copy()), dev(e1), dev(e2), ws, caches, ctx, n + 8)
    torch.cuda.synchronize()
    # oracle: the same composition
    want_p, pools = prefill_step(tokens[:, : n - 1], e1, layers, np.zeros(B))
    errs = twin_errors(lambda ds, ph: prefill_step(tokens[:, : n - 1], e1[:, ph], ds, np.zeros(B), dtype=np.float32)[0],
                       None, want_p, layers=layers)
    assert_twin_close(xp.cpu().numpy(), want_p, errs, "prefill step")

    def twin_start(ds, ph):
        # the fp32 evaluation's own prefill fills the caches its decode step reads
        _, own = prefill_step(tokens[:, : n - 1], e1[:, ph], ds, np.zeros(B), dtype=np.float32)
        for d, (kp, vp) in zip(ds, own):
            d.cache.k_pool, d.cache.v_pool = kp, vp
        return dual_flow_step(tokens[:, n - 1], e1[:, ph], e2[:, ph], ds, np.full(B, n - 1), dtype=np.float32)[0]

    done = []
    for Lc, (kp, vp) in zip(layers, pools):
        d = copy.copy(Lc)
        d.cache = copy.copy(Lc.cache)
        d.cache.k_pool, d.cache.v_pool = kp, vp
        done.append(d)
    want, _ = dual_flow_step(tokens[:, n - 1], e1, e2, done, np.full(B, n - 1))
    assert_twin_close(x_last.cpu().numpy(), want, twin_errors(twin_start, None, want, layers=layers),
                      "auxiliary start")


def check_prefill_chain(c, x, st, samples, tag):
    """Runs the prefill layer on chunk x [B][T][hidden] from positions st and checks every stage of
    the sampled rows (b, t) against the oracle applied to the GPU's own previous stage, read from
    the workspace (dfx_prefill_layer_taps): the normed rows' bf16 decisions, the whole Q/K/V
    projection row (fp32, accumulation bound), the appended key and value rows' decisions, the
    attention rows' decisions (GPU queries over the GPU's cache), the MLP's normed rows, the SwiGLU
    rows and the output rows (each projection within its accumulation bound). Returns the output."""
    B, T, H = x.shape
    Hq, Hkv, D, I = c.num_q_heads, c.num_kv_heads, c.head_dim, c.intermediate
    HqD, Nqkv = Hq * D, (Hq + 2 * Hkv) * D
    mc = int(st.max()) + T + 8
    cache = cache_of(c.cache)
    w = weights_of(c)
    ws = dfx.Workspace()
    xt = dev(x)
    print(f"prefill chain ({tag}): B={B} T={T} hidden={H}, {len(samples)} rows", flush=True)
    dfx.prefill_layer(xt, w, cache, dev(st), mc, workspace=ws)
    torch.cuda.synchronize()
    taps = dfx.prefill_layer_taps(w, cache, B, T, mc)
    buf = ws.buf.cpu().numpy()
    rows = np.array([b * T + t for b, t in samples])
    padded = -(-(B * T) // 64) * 64

    def bf16_region(name, K):
        return unpack_rows(buf[taps[name]: taps[name] + padded * K * 2].view(np.uint16), 1, B * T, K)[0, rows]

    h1, o, h2, inter = bf16_region("h1", H), bf16_region("o", HqD), bf16_region("h2", H), bf16_region("inter", I)
    qkv = buf[taps["q"]: taps["q"] + B * T * Nqkv * 4].view(np.float32).reshape(B * T, Nqkv)[rows]
    kp, vp = host_bits(cache.k), host_bits(cache.v)
    y = xt.cpu().numpy().reshape(B * T, H)[rows].astype(np.float64)
    x0 = x.reshape(B * T, H)[rows].astype(np.float64)
    absw = lambda m: np.abs(widen(m))
    same = {}
    # normed rows from the exact input
    h1_exact = rmsnorm(x0, c.g_attn, c.eps, rounded=False)
    same["h1"] = bf16_decisions_agree(h1, h1_exact, rel=1.0, scale=norm_bound(x0, 0 * x0, c.g_attn, h1_exact, c.eps))
    # the Q/K/V projection of the GPU's normed rows, and the appended key / value rows
    qkv_ref = grouped_linear(h1[None], c.w_qkv)[0]
    qkv_abs = absw(h1) @ absw(c.w_qkv).T
    assert np.all(np.abs(qkv - qkv_ref) <= gamma(H) * qkv_abs + 1e-30)
    tbl, bs = c.cache.block_table, c.cache.k_pool.shape[2]
    for i, (b, t) in enumerate(samples):
        pos = int(st[b]) + t
        for pool, lo in ((kp, HqD), (vp, HqD + Hkv * D)):
            got = pool[tbl[b, pos // bs], :, pos % bs, :].reshape(1, Hkv * D)
            same.setdefault("kv", []).append(bf16_decisions_agree(got, qkv_ref[i: i + 1, lo: lo + Hkv * D],
                                                                  rel=gamma(H), scale=qkv_abs[i: i + 1, lo: lo + Hkv * D]))
    same["kv"] = float(np.mean(same["kv"]))
    # attention rows: the GPU's queries over the GPU's cache
    o_exact = np.empty((len(samples), HqD))
    o_scale = np.empty_like(o_exact)
    G = Hq // Hkv
    for i, (b, t) in enumerate(samples):
        n = int(st[b]) + t + 1
        q = qkv[i, :HqD].reshape(1, Hq, D)
        o1, _, _, wts = decode_attention(q, None, None, 0, kp, vp, tbl[b: b + 1], np.array([n]), return_weights=True)
        o_exact[i] = o1.reshape(-1)
        K = widen(gather_kv(kp, tbl[b: b + 1], 0, n))
        V = widen(gather_kv(vp, tbl[b: b + 1], 0, n))
        for g in range(Hkv):
            for hh in range(G):
                h = g * G + hh
                o_scale[i, h * D:(h + 1) * D] = attention_row_bound(widen(q[0, h]), K[g], V[g], wts[(0, g)][hh], D)
    same["o"] = bf16_decisions_agree(o, o_exact, rel=1.0, scale=o_scale)
    # W_o and the residual (not kept), the MLP norm of that
    x1 = grouped_linear(o[None], c.w_o, residual=x0[None])[0]
    e1 = gamma(HqD) * (absw(o) @ absw(c.w_o).T) + U * np.abs(x1)
    h2_exact = rmsnorm(x1, c.g_mlp, c.eps, rounded=False)
    same["h2"] = bf16_decisions_agree(h2, h2_exact, rel=1.0, scale=norm_bound(x1, e1, c.g_mlp, h2_exact, c.eps))
    # gate/up with SwiGLU from the GPU's normed rows
    gu = grouped_linear(h2[None], c.w_gate_up)[0]
    gu_err = gamma(H) * (absw(h2) @ absw(c.w_gate_up).T)
    gate, up = gu[..., :I], gu[..., I:]
    sig = 1.0 / (1.0 + np.exp(-gate))
    e_int = 1.1 * gu_err[..., :I] * np.abs(up) + np.abs(gate * sig) * gu_err[..., I:] + 6 * U * np.abs(gate * sig * up)
    inter_exact = swiglu_couple(gu[None], None, rounded=False)[0]
    same["inter"] = bf16_decisions_agree(inter, inter_exact, rel=1.0, scale=e_int + U * np.abs(inter_exact))
    # W_down and the residual from the GPU's SwiGLU rows
    x2 = grouped_linear(inter[None], c.w_down, residual=x1[None])[0]
    bound = e1 + gamma(I) * (absw(inter) @ absw(c.w_down).T) + U * np.abs(x2)
    err = np.abs(y - x2)
    print("prefill chain: bf16 decisions equal to the oracle's:", {k: round(v, 5) for k, v in same.items()},
          "| output error / bound: max %.3g" % float((err / bound).max()), flush=True)
    assert np.all(err <= bound), float((err / bound).max())
    return xt


@pytest.mark.parametrize("B,T,start,shape,tiles", [
    # 3 x 50 rows from position 4: three 64-row groups with a ragged tail; every projection on the
    # 256 x 128 tile (hidden 288: Q/K/V 1536 features, W_o and W_down 288 = one full and one
    # ragged feature tile, gate/up 544 gate features = four full tiles of 128 and a ragged one;
    # down K = 17 k-steps)
    (3, 50, 4, dict(hidden=288, num_q_heads=8, num_kv_heads=2, head_dim=128, intermediate=544, w_std=0.05),
     "256 x 128"),
    # 2 x 3995 rows from position 0: gate/up, W_o and W_down on the 256 x 256 tile with a ragged
    # last row group (7990 rows) and ragged feature tiles
    (2, 3995, 0, dict(hidden=288, num_q_heads=4, num_kv_heads=2, head_dim=64, intermediate=1504, w_std=0.05),
     "256 x 256, ragged"),
    # the prefill benchmark's shape: 2 x 2048 rows, hidden 4096, 32/8 x 128, SwiGLU 14336 (gate/up,
    # W_o, W_down on the 256 x 256 tile, Q/K/V on the 192 x 256 one)
    (2, 2048, 0, dict(hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128, intermediate=14336, w_std=0.02),
     "benchmark shape"),
    # rows wider than the norm's 4096 register-resident values (hidden 5120: each row's last
    # 1024 values are read a second time)
    (2, 40, 3, dict(hidden=5120, num_q_heads=8, num_kv_heads=2, head_dim=128, intermediate=512, w_std=0.02),
     "wide rows"),
])
def test_prefill_layer_chain(B, T, start, shape, tiles):
    c = gen.layer_case(720 + T % 97, batch=B, context=start + 1, capacity=start + T + 8, **shape)
    x = np.random.default_rng(T).standard_normal((B, T, c.hidden)).astype(np.float32)
    st = np.full(B, start, np.int32)
    rng = np.random.default_rng(31)
    samples = [(0, 0), (0, T - 1), (B - 1, 0), (B - 1, T - 1), (B - 1, T // 2)]
    samples += [(int(b), int(t)) for b, t in zip(rng.integers(0, B, 11), rng.integers(0, T, 11))]
    check_prefill_chain(c, x, st, samples, tiles)
