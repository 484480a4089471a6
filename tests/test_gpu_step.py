"""GPU parity of the multi-layer decode step (dfx_dual_flow_decode_step)."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
import dual_flow_shared_amd as dfx
from gpu_util import cache_of, dev, host_bits
from oracle.step import dual_flow_step
from test_gpu_layer import weights_of
from twins import assert_twin_close, twin_errors

pytestmark = pytest.mark.gpu

KW = dict(vocab=300, batch=5, context=150, hidden=256, num_q_heads=8, num_kv_heads=2, head_dim=64,
          intermediate=512, w_std=0.05)


def inputs(c):
    layers = [weights_of(L) for L in c.layers]
    caches = [cache_of(L.cache) for L in c.layers]
    ctx = dev(c.layers[0].cache.context_lens + 1)
    return layers, caches, ctx, int(ctx.max()), dev(c.tokens), dev(c.embed_primary), dev(c.embed_aux)


def test_step_equals_layer_calls_bit_for_bit():
    """Embedding + norm in one kernel and each layer's down projection finished straight into
    the next layer's norm give exactly what one layer call per layer gives on the embedded rows."""
    c = gen.step_case(901, 3, **KW)
    layers, caches, ctx, maxc, tokens, e1, e2 = inputs(c)
    x = dfx.dual_flow_decode_step(tokens, e1, e2, layers, caches, ctx, maxc)
    ref_caches = [cache_of(L.cache) for L in c.layers]
    xr = torch.stack([e1[tokens.long()].float(), e2[tokens.long()].float()]).contiguous()
    for w, kv in zip(layers, ref_caches):
        dfx.dual_flow_decode_layer(xr, w, kv, ctx, maxc)
    torch.cuda.synchronize()
    assert torch.equal(x, xr)
    for a, b in zip(caches, ref_caches):      # bit patterns: the pools hold NaN poison
        assert np.array_equal(host_bits(a.k), host_bits(b.k)) and np.array_equal(host_bits(a.v), host_bits(b.v))


def test_step_sixteen_split_finish_equals_layer_calls():
    """The down projection's finish into the next layer's norm with 16 K splits (hidden 2048,
    SwiGLU 4096: 16 feature tiles of K = 4096) gives exactly what the layer calls give."""
    c = gen.step_case(902, 2, vocab=300, batch=4, context=120, hidden=2048, num_q_heads=16, num_kv_heads=4,
                      head_dim=128, intermediate=4096, w_std=0.03)
    layers, caches, ctx, maxc, tokens, e1, e2 = inputs(c)
    x = dfx.dual_flow_decode_step(tokens, e1, e2, layers, caches, ctx, maxc)
    ref_caches = [cache_of(L.cache) for L in c.layers]
    xr = torch.stack([e1[tokens.long()].float(), e2[tokens.long()].float()]).contiguous()
    for w, kv in zip(layers, ref_caches):
        dfx.dual_flow_decode_layer(xr, w, kv, ctx, maxc)
    torch.cuda.synchronize()
    assert torch.equal(x, xr)


def test_full_size_step_equals_layer_calls_bit_for_bit():
    """The decode step in the one-layer workload's shape and the benchmark's launch
    configuration (batch 32, context 8192, hidden 4096, 32/8 heads x 128, SwiGLU 14336, paged
    bf16 caches in permuted pools), three layers, seeded weights drawn on the device: the
    output rows and every cache equal one layer call per layer, bit for bit. Each layer is
    checked against the oracle at this size in the layer tests."""
    g = torch.Generator(device="cuda").manual_seed(77)
    B, H, Hq, Hkv, D, I, ctx_len, bs, vocab = 32, 4096, 32, 8, 128, 14336, 8192, 16, 1000

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)

    def unif(n, lo, hi):
        return torch.rand(n, generator=g, device="cuda") * (hi - lo) + lo

    layers, caches, refs = [], [], []
    nblk = B * ctx_len // bs
    for _ in range(3):
        layers.append(dfx.LayerWeights.from_row_major(
            unif(H, 0.9, 1.1), randn((Hq + 2 * Hkv) * D, H, std=0.02), randn(H, Hq * D, std=0.02),
            unif(H, 0.9, 1.1), randn(2 * I, H, std=0.02), randn(H, I, std=0.02), Hq, Hkv, D, 1e-5,
            unif(D, -1, 1), unif(I, -1, 1), unif(H, -1, 1)))
        table = torch.randperm(nblk, generator=g, device="cuda").to(torch.int32).view(B, ctx_len // bs)
        kv = dfx.KVCache(randn(nblk, Hkv, bs, D), randn(nblk, Hkv, bs, D), table)
        caches.append(kv)
        refs.append(dfx.KVCache(kv.k.clone(), kv.v.clone(), table))
    e1, e2 = randn(vocab, H), randn(vocab, H)
    tokens = torch.randint(0, vocab, (B,), generator=g, device="cuda", dtype=torch.int32)
    ctx = torch.full((B,), ctx_len, dtype=torch.int32, device="cuda")
    print("full-size step, 3 layers", flush=True)
    x = dfx.dual_flow_decode_step(tokens, e1, e2, layers, caches, ctx, ctx_len)
    xr = torch.stack([e1[tokens.long()].float(), e2[tokens.long()].float()]).contiguous()
    for w, kv in zip(layers, refs):
        dfx.dual_flow_decode_layer(xr, w, kv, ctx, ctx_len)
    torch.cuda.synchronize()
    assert torch.isfinite(x).all()
    assert torch.equal(x, xr)
    for a, b in zip(caches, refs):
        assert torch.equal(a.k.view(torch.int16), b.k.view(torch.int16))
        assert torch.equal(a.v.view(torch.int16), b.v.view(torch.int16))


def test_step_primary_only_and_against_the_oracle():
    c = gen.step_case(902, 2, **KW)
    layers, caches, ctx, maxc, tokens, e1, e2 = inputs(c)
    x = dfx.dual_flow_decode_step(tokens, e1, e2, layers, caches, ctx, maxc)
    k_dual = [host_bits(kv.k) for kv in caches]
    caches1 = [cache_of(L.cache) for L in c.layers]
    x1 = dfx.dual_flow_decode_step(tokens, e1, None, layers, caches1, ctx, maxc, n_flows=1)
    torch.cuda.synchronize()
    # the auxiliary flow changes neither the primary rows nor any cache byte
    assert torch.equal(x1[0], x[0])
    for a, kv in zip(k_dual, caches1):
        assert np.array_equal(a, host_bits(kv.k))
    before = c.layers[0].cache.context_lens
    want, pools = dual_flow_step(c.tokens, c.embed_primary, c.embed_aux, c.layers, before)
    errs = twin_errors(lambda ds, ph: dual_flow_step(c.tokens, c.embed_primary[:, ph], c.embed_aux[:, ph], ds, before,
                                                     dtype=np.float32)[0], None, want, layers=c.layers)
    assert_twin_close(x.cpu().numpy(), want, errs, "decode step")
    for (wk, _), got, L in zip(pools, k_dual, c.layers):
        # each layer's pool changes exactly at the primary's new slots, the oracle's too
        changed = np.argwhere(np.any(got != L.cache.k_pool, axis=-1))
        assert len(changed) == c.tokens.shape[0] * L.num_kv_heads
        assert np.array_equal(changed, np.argwhere(np.any(wk != L.cache.k_pool, axis=-1)))
    # layer 0 appends bf16 roundings of fp32 (GPU) and fp64 (oracle) projections of the same
    # normed rows: the same bits except next to a rounding midpoint
    assert (k_dual[0] != pools[0][0]).mean() < 1e-4


def test_step_graph_replays_match_eager():
    """The step allocates nothing and never synchronizes: captured once in a graph, every
    replay (with eager work and synchronizations in between) reproduces the eager result."""
    c = gen.step_case(903, 2, **KW)
    layers, caches, ctx, maxc, tokens, e1, e2 = inputs(c)
    B, H = c.tokens.shape[0], KW["hidden"]
    out = torch.empty(2, B, H, dtype=torch.float32, device="cuda")
    ws = dfx.Workspace()
    ws.get(dfx.step_workspace_size(layers, caches, B, 2, maxc))

    def step():
        dfx.dual_flow_decode_step(tokens, e1, e2, layers, caches, ctx, maxc, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    k_eager = [host_bits(kv.k) for kv in caches]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        for kv, k in zip(caches, k_eager):
            assert np.array_equal(host_bits(kv.k), k)
