"""Helpers for GPU tests: move seeded cases to the device, compare with the oracle."""
import numpy as np
import torch

import dual_flow_shared_amd as dfx


def dev(a, dtype=None):
    """numpy -> cuda tensor; uint16 arrays become bfloat16 tensors with the same bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host_bits(t):
    """cuda bfloat16 tensor -> numpy uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def cache_of(case):
    return dfx.KVCache(dev(case.k_pool), dev(case.v_pool),
                       None if case.block_table is None else dev(case.block_table))


def run_attn(case, cache=None, q2=True, a=True, num_splits=0, max_context=None, q1=None, q2v=None, ctx=None):
    cache = cache_of(case) if cache is None else cache
    ctx = dev(case.context_lens if ctx is None else ctx)
    mc = int(case.context_lens.max()) if max_context is None else max_context
    q1t = dev(case.q1 if q1 is None else q1)
    q2t = (dev(case.q2 if q2v is None else q2v) if q2 else None)
    at = dev(case.a) if (a and q2) else None
    o1, o2, lse = dfx.decode_attn(q1t, q2t, at, cache=cache, context_lens=ctx, max_context=mc,
                                  num_splits=num_splits)
    torch.cuda.synchronize()
    return (o1.cpu().numpy().astype(np.float64),
            None if o2 is None else o2.cpu().numpy().astype(np.float64),
            lse.cpu().numpy().astype(np.float64))


def max_err(a, b, rows=None):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if rows is not None:
        a, b = a[rows], b[rows]
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def lse_err(a, b):
    """max |a - b| over finite entries; -inf must match -inf."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    inf = np.isneginf(b)
    assert np.array_equal(np.isneginf(a), inf)
    return float(np.max(np.abs(a[~inf] - b[~inf]))) if (~inf).any() else 0.0


def bf16_decisions_agree(gpu_bits, oracle_fp64, rel=2e-6, scale=None):
    """bf16 outputs: the kernel's value g must be the bf16 rounding of some value within
    the kernel's arithmetic error (rel * scale, scale = magnitude of the operands that
    formed the value, default the value itself) of the oracle's exact value x:
    |g - x| <= rel * scale + ulp/2, ulp the bf16 spacing at max(|g|, |x|). Where x is not
    next to a rounding midpoint this forces equal bits. Returns the fraction of equal bits."""
    from oracle.numerics import bf16_bits, widen
    want = bf16_bits(oracle_fp64)
    got = np.asarray(gpu_bits, np.uint16)
    same = got == want
    if not same.all():
        x = np.asarray(oracle_fp64, np.float64)[~same]
        sc = np.abs(x) if scale is None else np.asarray(scale, np.float64)[~same]
        g = widen(got[~same])
        mag = np.maximum(np.abs(g), np.abs(x))
        _, e = np.frexp(np.where(mag > 0, mag, 1.0))
        half_ulp = np.ldexp(1.0, e - 9)                      # bf16: 8 significant bits
        ok = np.abs(g - x) <= rel * sc + half_ulp
        assert ok.all(), f"{(~ok).sum()} bf16 outputs farther from the exact value than rounding allows"
    return float(same.mean())


def unpack_rows(region, n_flows, batch, K):
    """[F][B][K] bf16 bits out of a region in the activation fragment order of the grouped
    linear (include/dfx.h, dfx_dual_flow_decode_layer_taps): pure index arithmetic."""
    R = 64 // n_flows
    f = np.arange(n_flows)[:, None, None]
    b = np.arange(batch)[None, :, None]
    k = np.arange(K)[None, None, :]
    g, q = b // R, f * R + b % R
    idx = ((((g * (K // 32) + k // 32) * 4 + q // 16) * 64 + q % 16 + 16 * ((k % 32) // 8)) * 8 + k % 8)
    return np.asarray(region)[idx]
