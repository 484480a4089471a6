"""One decode step of a stack of dual-flow layers (oracle, fp64).

What is computed (Sintesi Tecnica: Dual-Flow Transformers, "Architettura Core"): the two
flows take separate token embeddings and then pass through every layer with the layer's
shared matrices; the auxiliary flow runs at every generated position, and only the primary
writes each layer's cache. Reading where the pages are silent: the auxiliary row at a
generated position embeds that position's token -- the same id as the primary, looked up in
its own table -- since the pages name no other input for it. The step ends with the residual
rows after the last layer (the output head is not part of it).
"""
import numpy as np

from .layer import dual_flow_layer
from .numerics import widen


def embed(tokens, table_primary, table_aux=None):
    """x[0][b] = table_primary[tokens[b]], x[1][b] = table_aux[tokens[b]] (bf16 widened)."""
    tables = [table_primary] + ([table_aux] if table_aux is not None else [])
    return np.stack([widen(t)[np.asarray(tokens)] for t in tables])


def dual_flow_step(tokens, table_primary, table_aux, layers, context_lens_before, couple=True,
                   dtype=np.float64):
    """layers: LayerCase-like objects (weights, coupling vectors, cache with k_pool, v_pool,
    block_table). Applies dual_flow_layer layer by layer to the embedded rows, each layer
    appending to its own cache. Returns (x_out [F][B][hidden], [(k_pool', v_pool')])."""
    x = embed(tokens, table_primary, table_aux)
    pools = []
    for L in layers:
        kv = L.cache
        x, kp, vp, _ = dual_flow_layer(x, L.g_attn, L.g_mlp, L.w_qkv, L.w_o, L.w_gate_up, L.w_down,
                                       L.a if couple else None, L.b if couple else None,
                                       L.c if couple else None, L.eps, kv.k_pool, kv.v_pool,
                                       kv.block_table, context_lens_before, L.num_q_heads,
                                       L.num_kv_heads, L.head_dim, dtype=dtype)
        pools.append((kp, vp))
    return x, pools
