"""End-to-end parity bar of the layer-level calls: the GPU against an ensemble of fp32
evaluations of the oracle's own definition.

A decode or prefill layer rounds to bf16 at five points (normed rows, appended K/V, the
attention rows entering W_o, the MLP's normed rows and its intermediate). Any fp32
evaluation -- the GPU's, or the oracle evaluated in single precision -- lands next to a
rounding midpoint now and then and rounds to the other neighbour, which moves that row's
downstream outputs by a bf16 step times the weights. So the distance of an fp32 result from
the fp64 one is made of rare discrete steps, and which steps occur depends on the summation
orders.

The bar samples honest fp32 evaluations with different summation orders: the oracle in
float32 on the case itself and on copies whose hidden units, MLP units and head dimensions
are renumbered (a consistent permutation of the weights, vectors, rows and cache columns).
The exact result is the same up to that renumbering, only the order of every sum changes.
The GPU's max and median error from the fp64 oracle must stay within K_TWIN times the
largest max and median error of the ensemble (plus a floor of fp32 noise). K_TWIN = 2 allows
for the matrix cores' accumulation (blocks of 32 products added in sequence, where numpy
sums pairwise) and for a rounding step the ensemble does not happen to take; the GPU's
bf16 decisions are checked one by one, to their own bounds, by the per-stage chain checks.
"""
import copy

import numpy as np

K_TWIN = 2.0
N_TWINS = 8
FLOOR = 2.0 ** -20          # relative to the largest output magnitude: fp32 noise, no flip


def perms(c, t):
    """Renumbering t of the hidden units, MLP units and head dimensions (t = 0: none)."""
    H, I, D = c.hidden, c.intermediate, c.head_dim
    if t == 0:
        return np.arange(H), np.arange(I), np.arange(D)
    rng = np.random.default_rng([7919, t])
    return rng.permutation(H), rng.permutation(I), rng.permutation(D)


def permuted(c, ph, pi, pd):
    """A shallow copy of layer case ``c`` with hidden units renumbered by ph, MLP units by pi
    and head dimensions by pd (in every head of W_qkv's rows and W_o's columns, in the
    coupling vector a and in the cache pools' last axis)."""
    Hq, Hkv, D, I = c.num_q_heads, c.num_kv_heads, c.head_dim, c.intermediate
    rows = (np.arange(Hq + 2 * Hkv)[:, None] * D + pd[None, :]).reshape(-1)
    qcols = (np.arange(Hq)[:, None] * D + pd[None, :]).reshape(-1)
    d = copy.copy(c)
    d.x = c.x[..., ph]
    d.g_attn, d.g_mlp = c.g_attn[ph], c.g_mlp[ph]
    d.w_qkv = np.ascontiguousarray(c.w_qkv[rows][:, ph])
    d.w_o = np.ascontiguousarray(c.w_o[ph][:, qcols])
    d.w_gate_up = np.ascontiguousarray(np.concatenate([c.w_gate_up[:I][pi][:, ph], c.w_gate_up[I:][pi][:, ph]]))
    d.w_down = np.ascontiguousarray(c.w_down[ph][:, pi])
    d.a = None if c.a is None else c.a[..., pd]           # [D] or [Hq][D]
    d.b = None if c.b is None else c.b[pi]
    d.c = None if c.c is None else c.c[ph]
    kv = copy.copy(c.cache)
    kv.k_pool = np.ascontiguousarray(c.cache.k_pool[..., pd])
    kv.v_pool = np.ascontiguousarray(c.cache.v_pool[..., pd])
    d.cache = kv
    return d


def twin_errors(fn, c, exact, n=N_TWINS, layers=None):
    """Distances from ``exact`` of n fp32 evaluations: fn(cases, ph) runs the oracle in float32
    on the renumbered case(s) (one per layer when ``layers`` lists several cases, which share
    the hidden size and take the same renumbering) and returns outputs whose last axis is the
    renumbered hidden axis."""
    cases = [c] if layers is None else layers
    errs = []
    for t in range(n):
        ph, pi, pd = perms(cases[0], t)
        ds = [permuted(L, ph, pi, pd) for L in cases]
        y = np.asarray(fn(ds[0] if layers is None else ds, ph), np.float64)
        out = np.empty_like(y)
        out[..., ph] = y
        errs.append(np.abs(out - exact))
    return errs


def assert_twin_close(y, exact, errs, what="layer"):
    """The GPU's max and median distance from the fp64 result within K_TWIN times the
    ensemble's largest (plus the fp32-noise floor)."""
    e = np.abs(np.asarray(y, np.float64) - exact)
    tmax = max(float(x.max()) for x in errs)
    tmed = max(float(np.median(x)) for x in errs)
    floor = FLOOR * float(np.abs(exact).max())
    print(f"{what}: GPU vs fp64 max {e.max():.3g} median {np.median(e):.3g} | fp32 ensemble of {len(errs)}: "
          f"max {tmax:.3g} median {tmed:.3g} (plain fp32 twin: max {errs[0].max():.3g}) | "
          f"bars {K_TWIN * tmax + floor:.3g} / {K_TWIN * tmed + floor:.3g}", flush=True)
    assert e.max() <= K_TWIN * tmax + floor, (e.max(), tmax)
    assert np.median(e) <= K_TWIN * tmed + floor, (np.median(e), tmed)
