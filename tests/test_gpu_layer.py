"""GPU parity of one full dual-flow decode layer (dfx_dual_flow_decode_layer)."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
import dual_flow_shared_amd as dfx
from gpu_util import cache_of, dev, host_bits, max_err
from oracle.layer import dual_flow_layer
from oracle.numerics import widen

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


def layer_close(y, want, twin):
    """The layer rounds to bf16 at five points. Where a single-precision value and the
    fp64 value straddle a bf16 midpoint they round to neighbours, and with fp32
    accumulation over 4096-14336 terms about one element in a thousand does so; each
    flip moves downstream outputs by ulp * |w|. The yardstick is the oracle's own
    definition evaluated in float32 (`twin`): the kernel's distance from the fp64 oracle
    must be of the same size -- max within 3x and mean within 4x the twin's (matrix-core
    accumulation adds 32-term dot products sequentially, a little less accurately than a
    blocked BLAS sum, so slightly more values flip) -- and the median within 2e-3."""
    y, want, twin = (np.asarray(a, np.float64) for a in (y, want, twin))
    err, ref = np.abs(y - want), np.abs(twin - want)
    stats = dict(max=float(err.max()), mean=float(err.mean()), p50=float(np.median(err)),
                 twin_max=float(ref.max()), twin_mean=float(ref.mean()))
    print("layer error vs fp64 oracle:", stats)
    assert stats["max"] <= 3 * stats["twin_max"] + 1e-3, stats
    assert stats["mean"] <= 4 * stats["twin_mean"] + 1e-4, stats
    assert stats["p50"] < 2e-3, stats


SMALL = dict(batch=4, context=300, hidden=512, num_q_heads=8, num_kv_heads=2, head_dim=128,
             intermediate=1024, w_std=0.05)


def test_small_layer_parity_and_cache_diff():
    c = gen.layer_case(801, **SMALL)
    y, kp, vp = run_layer(c)
    want, wk, wv, mid = run_oracle(c)
    layer_close(y, want, run_oracle(c, dtype=np.float32)[0])
    # the pool changed exactly at the primary's new slots
    changed = np.argwhere(np.any(kp != c.cache.k_pool, axis=-1))
    assert len(changed) == c.batch * c.num_kv_heads
    assert np.array_equal(np.argwhere(np.any(wk != c.cache.k_pool, axis=-1)), changed)
    # appended rows are bf16 roundings of fp32 (GPU) and fp64 (oracle) projections: the same
    # bits except next to a rounding midpoint, where they are one bf16 step apart
    diff = kp != wk
    assert diff.mean() < 1e-4
    assert np.all(np.abs(widen(kp[diff]) - widen(wk[diff])) <= np.abs(widen(wk[diff])) * 2.0 ** -7)


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


def test_full_size_layer_sampled():
    c = gen.config_layer()
    y, kp, _ = run_layer(c)
    rows = [0, 31]
    want, wk, _, _ = run_oracle(c, batches=rows)
    twin = run_oracle(c, batches=rows, dtype=np.float32)[0]
    layer_close(y[:, rows], want[:, rows], twin[:, rows])
    assert np.all(np.isfinite(y))
    changed = np.argwhere(np.any(kp != c.cache.k_pool, axis=-1))
    assert len(changed) == c.batch * c.num_kv_heads
