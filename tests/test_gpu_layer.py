"""GPU parity of one full dual-flow decode layer (dfx_dual_flow_decode_layer)."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
import dual_flow_shared_amd as dfx
from gpu_util import bf16_decisions_agree, cache_of, dev, host_bits, unpack_rows
from oracle.attention import decode_attention, gather_kv
from oracle.layer import dual_flow_layer
from oracle.linear import grouped_linear, rmsnorm, swiglu_couple
from oracle.numerics import widen
from twins import assert_twin_close, twin_errors

pytestmark = pytest.mark.gpu


def weights_of(c, couple=True):
    return dfx.LayerWeights.from_row_major(dev(c.g_attn), dev(c.w_qkv), dev(c.w_o), dev(c.g_mlp), dev(c.w_gate_up),
                            dev(c.w_down), c.num_q_heads, c.num_kv_heads, c.head_dim, c.eps,
                            dev(c.a) if (couple and c.a is not None) else None,
                            dev(c.b) if (couple and c.b is not None) else None,
                            dev(c.c) if (couple and c.c is not None) else None)


def run_layer(c, flows=2, x=None, couple=True):
    cache = cache_of(c.cache)
    ctx = dev(c.cache.context_lens + 1)
    xt = dev((c.x if x is None else x)[:flows].copy())
    dfx.dual_flow_decode_layer(xt, weights_of(c, couple), cache, ctx, int(c.cache.context_lens.max()) + 1)
    torch.cuda.synchronize()
    return xt.cpu().numpy().astype(np.float64), host_bits(cache.k), host_bits(cache.v)


def run_oracle(c, flows=2, x=None, couple=True, batches=None, dtype=np.float64):
    kv = c.cache
    return dual_flow_layer((c.x if x is None else x)[:flows], c.g_attn, c.g_mlp, c.w_qkv, c.w_o,
                           c.w_gate_up, c.w_down, c.a if couple else None, c.b if couple else None,
                           c.c if couple else None, c.eps, kv.k_pool, kv.v_pool, kv.block_table,
                           kv.context_lens, c.num_q_heads, c.num_kv_heads, c.head_dim, batches=batches,
                           dtype=dtype)


def layer_close(c, y, flows=2, couple=True, rows=None, x=None, want=None):
    """End-to-end parity against the fp64 oracle on ``rows`` (all by default): within
    K_TWIN times the distance of an ensemble of fp32 evaluations of the oracle's definition
    (tests/twins.py). Returns the fp64 result."""
    sel = slice(None) if rows is None else list(rows)
    if want is None:
        want = run_oracle(c, flows, x=x, couple=couple, batches=rows)[0]
    exact = want[:, sel]
    errs = twin_errors(lambda d, ph: run_oracle(d, flows, x=None if x is None else x[..., ph], couple=couple,
                                                batches=rows, dtype=np.float32)[0][:, sel], c, exact)
    assert_twin_close(np.asarray(y)[:, sel], exact, errs)
    return want


U = 2.0 ** -24                 # fp32 unit roundoff
SPLIT = 0.0                    # the layer's attention splits its fp32 Q and P into three bf16
                               # terms, which hold every fp32 bit: no split error


def gamma(k):
    """Accumulation bound of a k-term fp32 dot product on the matrix cores: 32-term MFMA
    blocks added in sequence over k / 32 steps, plus the split-K partial sums and the
    residual add (a few more roundings)."""
    return (k / 32 + 64) * U


def norm_bound(xin, err_in, gain, y, eps):
    """Error bound of y = x r g (RMSNorm before its bf16 rounding): the input's error (through x
    and through r) and the fp32 norm (sum of squares over H terms, reciprocal square root, two
    products)."""
    H = xin.shape[-1]
    r = 1.0 / np.sqrt(np.mean(xin * xin, axis=-1, keepdims=True) + eps)
    rel_r = np.linalg.norm(err_in, axis=-1, keepdims=True) / np.linalg.norm(xin, axis=-1, keepdims=True)
    return np.abs(widen(gain)) * r * (err_in + np.abs(xin) * (rel_r + (H / 2 + 8) * U)) + 4 * U * np.abs(y)


def attention_row_bound(q, K, V, w, D):
    """Error bound of one attention row (query q, keys K [n][D], values V, exact weights w):
    score error max_p scale sum|q||k| (D/32 + 64) u (Q and P are split into bf16 terms exactly),
    doubled through the softmax, plus (n/32 + 64) u, times sum_p w_p |v_p|."""
    n = K.shape[0]
    sabs = np.abs(q) @ np.abs(K).T / np.sqrt(D)
    ds = sabs.max() * (SPLIT + (D / 32 + 64) * U)
    rel = 2 * ds + 2 * SPLIT + (n / 32 + 64) * U
    return rel * (w @ np.abs(V))


def check_layer_chain(c, flows=2, couple=True, rows=None):
    """Runs the layer and checks every stage against the oracle applied to the GPU's own
    previous stage (read from the workspace through dfx_dual_flow_decode_layer_taps): each
    fp32 value within its accumulation bound, and every bf16 rounding decision (R1 normed
    rows, R2 appended K/V, R3 attention rows, R4 normed rows, R5 SwiGLU rows) the rounding of
    a value within that bound of the oracle's exact one. Returns (x_out, k pool, v pool)."""
    F, B = flows, c.batch
    H, Hq, Hkv, D = c.g_attn.shape[0], c.num_q_heads, c.num_kv_heads, c.head_dim
    I = c.w_down.shape[1]
    HqD, Nqkv = Hq * D, (Hq + 2 * Hkv) * D
    rows = np.arange(B) if rows is None else np.asarray(rows)
    cache = cache_of(c.cache)
    ctx_after = c.cache.context_lens + 1
    maxc = int(ctx_after.max())
    xt = dev(c.x[:F].copy())
    w = weights_of(c, couple)
    ws = dfx.Workspace()
    dfx.dual_flow_decode_layer(xt, w, cache, dev(ctx_after), maxc, workspace=ws)
    torch.cuda.synchronize()
    taps = dfx.layer_taps(w, cache, B, F, maxc)
    buf = ws.buf.cpu().numpy()
    padded = -(-B // (64 // F)) * 64

    def bf16_region(name, K):
        r = buf[taps[name]: taps[name] + padded * K * 2].view(np.uint16)
        return unpack_rows(r, F, B, K)[:, rows]

    h1, o, h2, inter = bf16_region("h1", H), bf16_region("o", HqD), bf16_region("h2", H), bf16_region("inter", I)
    q = buf[taps["q"]: taps["q"] + F * B * Nqkv * 4].view(np.float32).reshape(F, B, Nqkv)[:, rows, :HqD]
    x_out = xt.cpu().numpy().astype(np.float64)
    kp, vp = host_bits(cache.k), host_bits(cache.v)
    x0 = widen(c.x[:F][:, rows])
    a_vec, b_vec, c_vec = (c.a, c.b, c.c) if (couple and F == 2) else (None, None, None)
    absw = lambda m: np.abs(widen(m))

    def norm_scale(xin, err_in, gain, y):
        return norm_bound(xin, err_in, gain, y, c.eps)

    # R1: normed rows from the exact input
    h1_exact = rmsnorm(x0, c.g_attn, c.eps, rounded=False)
    same = {"h1": bf16_decisions_agree(h1, h1_exact, rel=1.0, scale=norm_scale(x0, 0 * x0, c.g_attn, h1_exact))}
    # Q columns (fp32) and the appended K/V rows (R2) from the GPU's normed rows
    qkv_ref = grouped_linear(h1, c.w_qkv)
    qkv_abs = absw(h1) @ absw(c.w_qkv).T
    assert np.all(np.abs(q - qkv_ref[..., :HqD]) <= gamma(H) * qkv_abs[..., :HqD] + 1e-30)
    kv = c.cache
    pos = kv.context_lens[rows]
    blk = kv.block_table[rows, pos // kv.k_pool.shape[2]]
    slot = pos % kv.k_pool.shape[2]
    for pool, lo in ((kp, HqD), (vp, HqD + Hkv * D)):
        got = pool[blk, :, slot, :].reshape(len(rows), Hkv * D)
        same["kv%d" % lo] = bf16_decisions_agree(got, qkv_ref[0, :, lo: lo + Hkv * D], rel=gamma(H),
                                                 scale=qkv_abs[0, :, lo: lo + Hkv * D])
    # R3: attention rows from the GPU's queries and the GPU's cache
    q1 = q[0].reshape(len(rows), Hq, D)
    q2 = q[1].reshape(len(rows), Hq, D) if F == 2 else None
    sub = lambda t: t[rows]
    o1, o2, _, wts = decode_attention(q1, q2, a_vec, 0, kp, vp, sub(kv.block_table), sub(ctx_after), return_weights=True)
    o_exact = np.stack([o1] + ([o2] if F == 2 else [])).reshape(F, len(rows), HqD)
    o_scale = np.zeros_like(o_exact)
    G = Hq // Hkv
    Qs = [q1] + ([q2 + widen(a_vec) * q1 if a_vec is not None else q2] if F == 2 else [])
    for i, b in enumerate(rows):
        n = int(ctx_after[b])
        K = widen(gather_kv(kp, kv.block_table[rows], i, n))
        V = widen(gather_kv(vp, kv.block_table[rows], i, n))
        for g in range(Hkv):
            Wt = wts[(i, g)]                                                  # [F*G][n]
            for f in range(F):
                for hh in range(G):
                    h = g * G + hh
                    o_scale[f, i, h * D:(h + 1) * D] = attention_row_bound(Qs[f][i, h], K[g], V[g], Wt[f * G + hh], D)
    same["o"] = bf16_decisions_agree(o, o_exact, rel=1.0, scale=o_scale)
    # x1 (not kept by the layer) from the GPU's attention rows, R4 from it
    wo_abs = absw(o) @ absw(c.w_o).T
    x1 = grouped_linear(o, c.w_o, residual=x0)
    e1 = gamma(HqD) * wo_abs + U * np.abs(x1)
    h2_exact = rmsnorm(x1, c.g_mlp, c.eps, rounded=False)
    same["h2"] = bf16_decisions_agree(h2, h2_exact, rel=1.0, scale=norm_scale(x1, e1, c.g_mlp, h2_exact))
    # R5 from the GPU's normed rows
    gu = grouped_linear(h2, c.w_gate_up)
    gu_err = gamma(H) * (absw(h2) @ absw(c.w_gate_up).T)
    gate, up = gu[..., :I], gu[..., I:]
    sig = 1.0 / (1.0 + np.exp(-gate))
    e_int = 1.1 * gu_err[..., :I] * np.abs(up) + np.abs(gate * sig) * gu_err[..., I:] + 6 * U * np.abs(gate * sig * up)
    if b_vec is not None:
        e_int[1] = e_int[1] + np.abs(widen(b_vec)) * e_int[0]
    inter_exact = swiglu_couple(gu, b_vec, rounded=False)
    same["inter"] = bf16_decisions_agree(inter, inter_exact, rel=1.0, scale=e_int + U * np.abs(inter_exact))
    # output rows from the GPU's SwiGLU rows
    m_abs = absw(inter) @ absw(c.w_down).T
    if c_vec is not None:
        m_abs[1] = m_abs[1] + np.abs(widen(c_vec)) * m_abs[0]
    x2 = grouped_linear(inter, c.w_down, couple=c_vec, residual=x1)
    bound = e1 + gamma(I) * m_abs + U * np.abs(x2)
    err = np.abs(x_out[:, rows] - x2)
    print("chain: bf16 decisions equal to the oracle's:", {k: round(v, 5) for k, v in same.items()},
          "| output error / bound: max %.3g" % float((err / bound).max()))
    assert np.all(err <= bound), float((err / bound).max())
    return x_out, kp, vp


SMALL = dict(batch=4, context=300, hidden=512, num_q_heads=8, num_kv_heads=2, head_dim=128,
             intermediate=1024, w_std=0.05)


def test_small_layer_parity_and_cache_diff():
    c = gen.layer_case(801, **SMALL)
    y, kp, vp = check_layer_chain(c)
    want, wk, wv, mid = run_oracle(c)
    layer_close(c, y, want=want)
    # the pool changed exactly at the primary's new slots
    changed = np.argwhere(np.any(kp != c.cache.k_pool, axis=-1))
    assert len(changed) == c.batch * c.num_kv_heads
    assert np.array_equal(np.argwhere(np.any(wk != c.cache.k_pool, axis=-1)), changed)


@pytest.mark.parametrize("seed", [804, 805])
def test_layer_two_row_groups(seed):
    # 40 sequences of two flows fill two 64-row groups of the projections (the second one
    # partly), with head_dim 64
    c = gen.layer_case(seed, batch=40, context=200, hidden=256, num_q_heads=4, num_kv_heads=2,
                       head_dim=64, intermediate=512, w_std=0.05)
    y, _, _ = check_layer_chain(c)
    layer_close(c, y)
    y1, _, _ = check_layer_chain(c, flows=1)
    assert np.array_equal(y1[0], y[0])


@pytest.mark.parametrize("heads,block", [((32, 2), 16), ((8, 2), 8)])
def test_layer_vector_attention_path(heads, block):
    # 32 query rows per KV head (both flows, GQA 16), or 8-token blocks: the attention runs on
    # the vector path
    c = gen.layer_case(807, batch=3, context=100, hidden=256, num_q_heads=heads[0], num_kv_heads=heads[1],
                       head_dim=64, intermediate=256, block_size=block, w_std=0.05)
    y, _, _ = check_layer_chain(c)
    layer_close(c, y)


def test_layer_primary_only_chain():
    c = gen.layer_case(806, **SMALL)
    check_layer_chain(c, flows=1)
    check_layer_chain(c, flows=2, couple=False)


def test_aux_never_changes_primary_or_cache():
    c = gen.layer_case(802, **SMALL)
    y2, k2, v2 = run_layer(c, flows=2)
    y1, k1, v1 = run_layer(c, flows=1)
    assert np.array_equal(y2[0], y1[0]) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    other = c.x.copy()
    other[1] = other[1] * -2 + 0.5
    y3, k3, _ = run_layer(c, x=other)
    assert np.array_equal(y3[0], y2[0]) and np.array_equal(k3, k2)


def test_aux_equals_primary_without_coupling():
    c = gen.layer_case(803, **SMALL)
    x = np.stack([c.x[0], c.x[0]])
    y, _, _ = run_layer(c, x=x, couple=False)
    assert np.array_equal(y[0], y[1])


def test_full_size_layer_all_rows():
    """The one-layer workload at full size (batch 32 x context 8192, hidden 4096, SwiGLU 14336):
    every stage of all 32 sequences of both flows against the oracle, and the end-to-end rows
    against the fp32 ensemble."""
    c = gen.config_layer()
    print("full-size layer: chain check over all 32 sequences", flush=True)
    y, kp, _ = check_layer_chain(c)
    layer_close(c, y)
    assert np.all(np.isfinite(y))
    changed = np.argwhere(np.any(kp != c.cache.k_pool, axis=-1))
    assert len(changed) == c.batch * c.num_kv_heads


@pytest.mark.parametrize("shape", [dict(hidden=2048, num_q_heads=32, num_kv_heads=8, intermediate=4096),
                                   dict(hidden=4096, num_q_heads=8, num_kv_heads=4, intermediate=1024)])
def test_layer_sixteen_split_finishes(shape):
    """Shapes whose projections split K 16 ways, so the finish kernels sum their tiles in the
    16-split form: hidden 2048 with 32 query heads (W_o and W_down over 16 feature tiles of
    K = 4096: 16 splits each), and hidden 4096 with 8/4 heads (the Q/K/V projection's 2048
    outputs over K = 4096: 16 splits)."""
    c = gen.layer_case(809, batch=4, context=300, head_dim=128, w_std=0.03, **shape)
    y, _, _ = check_layer_chain(c)
    layer_close(c, y)
    y1, _, _ = check_layer_chain(c, flows=1)
    assert np.array_equal(y1[0], y[0])


@pytest.mark.parametrize("flows", [2, 1])
def test_layer_single_sequence(flows):
    # one sequence: a 64-row group holding one row per flow, context 1 (the appended token only)
    c = gen.layer_case(806, batch=1, context=1, hidden=256, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       intermediate=512, w_std=0.05)
    y, kp, _ = check_layer_chain(c, flows=flows)
    layer_close(c, y, flows=flows)
    assert np.sum(np.any(kp != c.cache.k_pool, axis=-1)) == c.num_kv_heads


def test_layer_clamps_context_lengths_like_the_attention():
    """Context lengths above max_context attend max_context positions and append the new row at
    position max_context - 1 (the same clamping as the attention's, so the appended row is one
    the step attends); a negative length acts as 0: nothing attended, the row appended at
    position 0."""
    c = gen.layer_case(808, **SMALL)
    maxc = int(c.cache.context_lens.max()) + 1
    w = weights_of(c)

    def run(ctx):
        cache = cache_of(c.cache)
        x = dev(c.x.copy())
        dfx.dual_flow_decode_layer(x, w, cache, dev(np.asarray(ctx, np.int32)), maxc)
        torch.cuda.synchronize()
        return x.cpu().numpy(), host_bits(cache.k), host_bits(cache.v)

    base = c.cache.context_lens + 1
    wild, tame = base.copy(), base.copy()
    wild[0], tame[0] = maxc + 7, maxc
    wild[1], tame[1] = -3, 0
    for got, want in zip(run(wild), run(tame)):
        assert np.array_equal(got, want)
