"""Graph capture of the output head, the MoE block and the prefill layer: each allocates nothing
inside the library and never synchronizes, so a captured call replays the eager result bit for
bit (four replays, with eager work and synchronizations in between, inputs reset eagerly)."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
import dual_flow_shared_amd as dfx
from gpu_util import cache_of, dev, host_bits

pytestmark = pytest.mark.gpu


def capture(fn):
    """Warm up fn on a side stream, then capture it; returns (graph, outputs of the capture)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    return graph, outs


def test_output_head_graph_replays():
    c = gen.head_case(930, 2, 24, 512, 4112, w_std=0.3)
    x, g, w = dev(c.x), dev(c.gain), dfx.pack_weight(dev(c.w_out))
    noise = dev(c.noise)
    ws = dfx.Workspace()
    ws.get(dfx.output_head_workspace_size(2, 24, 512, 4112))
    call = lambda: dfx.output_head(x, g, c.eps, w, noise, want_p_mix=True, workspace=ws)
    tok_e, a_e, p_e = call()
    torch.cuda.synchronize()
    tok_e, a_e, p_e = tok_e.clone(), a_e.clone(), p_e.clone()
    graph, (tok, alpha, pm) = capture(call)
    for _ in range(4):
        tok.fill_(-7)
        pm.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(tok, tok_e) and torch.equal(alpha, a_e) and torch.equal(pm, p_e)


def test_moe_block_graph_replays():
    c = gen.moe_case(931, 20, hidden=256, num_experts=8, intermediate=256, router_std=0.3, w_std=0.05)
    w = dfx.MoeWeights.from_row_major(dev(c.gain), dev(c.w_router), dev(c.w_gate_up), dev(c.w_down), 2, 3, c.eps,
                                      dev(c.b), dev(c.c))
    x0 = dev(c.x)
    x = x0.clone()
    ws = dfx.Workspace()
    ws.get(dfx.moe_workspace_size(w, 20, 2))
    dfx.moe_mlp(x, w, workspace=ws)
    torch.cuda.synchronize()
    eager = x.clone()
    x.copy_(x0)
    graph, _ = capture(lambda: dfx.moe_mlp(x, w, workspace=ws))
    for _ in range(4):
        x.copy_(x0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(x, eager)


def test_prefill_layer_graph_replays():
    B, start, T = 2, 5, 70
    c = gen.layer_case(932, batch=B, context=start + 1, capacity=start + T + 8, hidden=256, num_q_heads=8,
                       num_kv_heads=2, head_dim=128, intermediate=512, w_std=0.05)
    w = dfx.LayerWeights.from_row_major(dev(c.g_attn), dev(c.w_qkv), dev(c.w_o), dev(c.g_mlp), dev(c.w_gate_up),
                                        dev(c.w_down), c.num_q_heads, c.num_kv_heads, c.head_dim, c.eps)
    cache = cache_of(c.cache)
    st = dev(np.full(B, start, np.int32))
    x0 = dev(np.random.default_rng(6).standard_normal((B, T, c.hidden)).astype(np.float32))
    x = x0.clone()
    ws = dfx.Workspace()
    dfx.prefill_layer(x, w, cache, st, start + T + 8, workspace=ws)
    torch.cuda.synchronize()
    eager, k_eager = x.clone(), host_bits(cache.k)
    x.copy_(x0)
    graph, _ = capture(lambda: dfx.prefill_layer(x, w, cache, st, start + T + 8, workspace=ws))
    for _ in range(4):
        x.copy_(x0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(x, eager) and np.array_equal(host_bits(cache.k), k_eager)
