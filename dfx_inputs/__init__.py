"""Seeded synthetic inputs for the dual-flow decode path.

This module draws random numbers and lays them out in the buffers that the
library and the oracle both read: query rows, the paged or contiguous K/V
pool with its block table, coupling vectors, layer weights and residual rows.
It holds no step of the method's arithmetic (no attention, coupling, norm or
linear); the only numeric operation here is the fp32 -> bf16 conversion that
turns an fp32 draw into a bf16 input.

Every tensor is drawn from its own PCG64 sub-stream keyed by
(seed, tensor id, indices), so any slice (one sequence, one KV head) can be
regenerated alone and large pools fill in parallel threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_QNAN = 0x7FC0  # quiet NaN bit pattern used to poison unreferenced cache slots

# tensor ids of the sub-streams
TID_Q1, TID_Q2, TID_A, TID_K, TID_V, TID_CTX, TID_PERM = 1, 2, 3, 4, 5, 6, 7
TID_X1, TID_X2, TID_WQKV, TID_WO, TID_WGU, TID_WD = 11, 12, 13, 14, 15, 16
TID_G1, TID_G2, TID_B, TID_C = 17, 18, 19, 20
TID_LIN_X, TID_LIN_W, TID_LIN_CPL, TID_LIN_RES = 21, 22, 23, 24
TID_TOK, TID_E1, TID_E2 = 31, 32, 33
TID_HX, TID_HG, TID_WOUT, TID_NOISE = 41, 42, 43, 44
TID_MX, TID_MG, TID_WR, TID_WEGU, TID_WED, TID_MB, TID_MC = 51, 52, 53, 54, 55, 56, 57


def stream(seed: int, tid: int, *idx: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tid), *[int(i) for i in idx]])


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaN -> quiet NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = BF16_QNAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seed, tid, idx, shape, scale=1.0):
    x = stream(seed, tid, *idx).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _uniform(seed, tid, idx, shape, lo, hi):
    return stream(seed, tid, *idx).uniform(lo, hi, size=shape).astype(np.float32)


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


@dataclass
class AttnCase:
    """One decode-attention problem: queries, coupling vector and a K/V pool."""
    seed: int
    dtype: str                      # element type of q1/q2 and the pool: "f32" or "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int                 # tokens per block (paged) or capacity per sequence (contiguous)
    paged: bool
    context_lens: np.ndarray        # int32 [B]
    block_table: Optional[np.ndarray]  # int32 [B][max_blocks] or None (contiguous)
    k_pool: np.ndarray              # [num_blocks][Hkv][block_size][D], float32 or uint16 bits
    v_pool: np.ndarray
    q1: np.ndarray                  # [B][Hq][D]
    q2: np.ndarray                  # [B][Hq][D] (raw auxiliary query W_q x2)
    a: np.ndarray                   # float32 [D] (a_head_stride 0) or [Hq][D] (stride D)
    a_head_stride: int
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])


def _fill_pool(pool, seed, tid, dtype, ctx, table, bs, paged, D, workers):
    """Write the logical rows of every (b, g) into the pool through the table."""
    B, Hkv = len(ctx), pool.shape[1]

    def one(bg):
        b, g = bg
        n = int(ctx[b])
        if n == 0:
            return
        rows = _as_dtype(_normal(seed, tid, (b, g), (n, D)), dtype)
        if not paged:
            pool[b, g, :n] = rows
            return
        nblk = -(-n // bs)
        full = (n // bs) * bs
        blocks = table[b, :nblk]
        if full:
            pool[blocks[: n // bs], g] = rows[:full].reshape(n // bs, bs, D)
        if full < n:
            pool[blocks[-1], g, : n - full] = rows[full:]

    jobs = [(b, g) for b in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, jobs))


def attention_case(seed: int, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   context_lens, dtype: str = "bf16", paged: bool = True, block_size: int = 16,
                   num_blocks: Optional[int] = None, capacity: Optional[int] = None,
                   a_per_head: bool = False, poison: bool = True,
                   workers: Optional[int] = None) -> AttnCase:
    """Build a seeded decode-attention case.

    Queries, K and V ~ N(0, 1); the coupling vector a ~ U(-1, 1) per head_dim
    (or per (head, head_dim) when ``a_per_head``). Paged pools take a seeded
    permutation of the block ids, each sequence a consecutive slice of it;
    table entries past a sequence's last block and every unreferenced slot are
    filled with poison (NaN values; a spare poisoned block id in the table). With
    ``capacity`` every sequence owns the blocks of that many tokens.
    """
    ctx = np.asarray(context_lens, dtype=np.int32).reshape(batch)
    D, Hkv = head_dim, num_kv_heads
    workers = workers or _workers()
    el = np.float32 if dtype == "f32" else np.uint16
    fill = (np.float32(np.nan) if dtype == "f32" else np.uint16(BF16_QNAN)) if poison else 0
    if paged:
        # every sequence owns the blocks of its context, or of ``capacity`` tokens if that is
        # more (room for appends; those slots hold poison until written)
        nblk = [max(-(-int(n) // block_size), 0 if capacity is None else -(-capacity // block_size))
                for n in ctx]
        need = sum(nblk)
        nb = num_blocks if num_blocks is not None else need + 1
        if nb < need:
            raise ValueError(f"pool of {nb} blocks cannot hold {need}")
        perm = stream(seed, TID_PERM).permutation(nb).astype(np.int32)
        width = max(1, max(nblk) if capacity is None else -(-capacity // block_size))
        spare = int(perm[need]) if nb > need else int(perm[0])
        table = np.full((batch, width), spare, dtype=np.int32)
        off = 0
        for b, k in enumerate(nblk):
            table[b, :k] = perm[off:off + k]
            off += k
        shape = (nb, Hkv, block_size, D)
        bs = block_size
    else:
        cap = capacity if capacity is not None else max(1, int(ctx.max()))
        table = None
        shape = (batch, Hkv, cap, D)
        bs = cap
    k_pool = np.empty(shape, dtype=el)
    v_pool = np.empty(shape, dtype=el)
    k_pool.fill(fill)
    v_pool.fill(fill)
    _fill_pool(k_pool, seed, TID_K, dtype, ctx, table, bs, paged, D, workers)
    _fill_pool(v_pool, seed, TID_V, dtype, ctx, table, bs, paged, D, workers)
    q1 = _as_dtype(_normal(seed, TID_Q1, (), (batch, num_q_heads, D)), dtype)
    q2 = _as_dtype(_normal(seed, TID_Q2, (), (batch, num_q_heads, D)), dtype)
    if a_per_head:
        a = _uniform(seed, TID_A, (), (num_q_heads, D), -1.0, 1.0)
        stride = D
    else:
        a = _uniform(seed, TID_A, (), (D,), -1.0, 1.0)
        stride = 0
    return AttnCase(seed, dtype, batch, num_q_heads, num_kv_heads, D, bs, paged, ctx, table,
                    k_pool, v_pool, q1, q2, a, stride)


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence context lengths uniform in [lo, hi] (inclusive)."""
    return stream(seed, TID_CTX).integers(lo, hi + 1, size=batch).astype(np.int32)


# ---------------------------------------------------------------- linear / layer

@dataclass
class LinearCase:
    seed: int
    n_flows: int
    rows: int
    in_features: int
    out_features: int
    x: np.ndarray          # [F][rows][K] float32 or uint16 bits (x_dtype)
    x_dtype: str
    w: np.ndarray          # [N][K] uint16 bits
    couple: Optional[np.ndarray]    # float32 [N] or None
    residual: Optional[np.ndarray]  # float32 [F][rows][N] or None


def linear_case(seed: int, n_flows: int, rows: int, in_features: int, out_features: int,
                x_dtype: str = "bf16", w_std: float = 0.02, with_couple: bool = False,
                with_residual: bool = False) -> LinearCase:
    x = _normal(seed, TID_LIN_X, (), (n_flows, rows, in_features))
    w = f32_to_bf16_bits(_normal(seed, TID_LIN_W, (), (out_features, in_features), w_std))
    cpl = _uniform(seed, TID_LIN_CPL, (), (out_features,), -1.0, 1.0) if with_couple else None
    res = _normal(seed, TID_LIN_RES, (), (n_flows, rows, out_features)) if with_residual else None
    return LinearCase(seed, n_flows, rows, in_features, out_features, _as_dtype(x, x_dtype), x_dtype,
                      w, cpl, res)


def _bf16_matrix(seed, tid, n, k, std, workers):
    """[n][k] bf16 bits ~ N(0, std), in row blocks of 512 with sub-streams (seed, tid, first
    row) so that large matrices fill in parallel."""
    out = np.empty((n, k), dtype=np.uint16)
    step = 512

    def one(r0):
        r1 = min(n, r0 + step)
        out[r0:r1] = f32_to_bf16_bits(_normal(seed, tid, (r0,), (r1 - r0, k), std))

    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(0, n, step)))
    return out


@dataclass
class LayerCase:
    """One dual-flow decode layer: weights, coupling vectors, residual rows and a paged cache."""
    seed: int
    batch: int
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    intermediate: int
    eps: float
    x: np.ndarray           # float32 [2][B][hidden]: flow 0 primary, flow 1 auxiliary
    g_attn: np.ndarray      # float32 [hidden]
    g_mlp: np.ndarray       # float32 [hidden]
    w_qkv: np.ndarray       # uint16 [(Hq + 2 Hkv) D][hidden]
    w_o: np.ndarray         # uint16 [hidden][Hq D]
    w_gate_up: np.ndarray   # uint16 [2 I][hidden]: gate rows, then up rows
    w_down: np.ndarray      # uint16 [hidden][I]
    a: Optional[np.ndarray]  # float32 [D] or None
    b: Optional[np.ndarray]  # float32 [I] or None
    c: Optional[np.ndarray]  # float32 [hidden] or None
    cache: AttnCase          # pool with ctx-1 filled tokens; the slot at ctx-1 is poison


def layer_case(seed: int, batch: int, context: int, hidden: int, num_q_heads: int,
               num_kv_heads: int, head_dim: int, intermediate: int, couple: bool = True,
               num_blocks: Optional[int] = None, block_size: int = 16, w_std: float = 0.02,
               eps: float = 1e-5, workers: Optional[int] = None,
               capacity: Optional[int] = None) -> LayerCase:
    """Seeded config of one layer: weights ~ N(0, w_std) bf16, residual rows ~ N(0, 1),
    norm gains ~ U(0.9, 1.1), coupling vectors ~ U(-1, 1); the cache holds
    ``context - 1`` pre-filled tokens per sequence so the step's append makes
    ``context`` attended positions. ``capacity`` (default ``context``) sizes each sequence's
    blocks, so a prompt chunk can be appended past the pre-filled tokens."""
    workers = workers or _workers()
    D, I, Hq, Hkv = head_dim, intermediate, num_q_heads, num_kv_heads
    cache = attention_case(seed, batch, Hq, Hkv, D, np.full(batch, context - 1, np.int32), "bf16",
                           paged=True, block_size=block_size, num_blocks=num_blocks,
                           capacity=capacity or context, workers=workers)
    x = np.stack([_normal(seed, TID_X1, (), (batch, hidden)), _normal(seed, TID_X2, (), (batch, hidden))])

    def wmat(tid, n, k):
        return _bf16_matrix(seed, tid, n, k, w_std, workers)

    w_qkv = wmat(TID_WQKV, (Hq + 2 * Hkv) * D, hidden)
    w_o = wmat(TID_WO, hidden, Hq * D)
    w_gu = wmat(TID_WGU, 2 * I, hidden)
    w_d = wmat(TID_WD, hidden, I)
    g1 = _uniform(seed, TID_G1, (), (hidden,), 0.9, 1.1)
    g2 = _uniform(seed, TID_G2, (), (hidden,), 0.9, 1.1)
    a = _uniform(seed, TID_A, (1,), (D,), -1.0, 1.0) if couple else None
    b = _uniform(seed, TID_B, (), (I,), -1.0, 1.0) if couple else None
    c = _uniform(seed, TID_C, (), (hidden,), -1.0, 1.0) if couple else None
    return LayerCase(seed, batch, hidden, Hq, Hkv, D, I, eps, x, g1, g2, w_qkv, w_o, w_gu, w_d,
                     a, b, c, cache)


# ------------------------------------------------------------- named workloads

@dataclass
class StepCase:
    """A stack of dual-flow layers with their own caches, both flows' token embedding tables and
    the token ids at the generated position."""
    seed: int
    tokens: np.ndarray          # int32 [B]
    embed_primary: np.ndarray   # uint16 [vocab][hidden]
    embed_aux: np.ndarray       # uint16 [vocab][hidden]: the auxiliary flow's own table
    layers: list                # LayerCase per layer (its residual rows x are unused)


def step_case(seed: int, n_layers: int, vocab: int, batch: int, context: int, hidden: int,
              num_q_heads: int, num_kv_heads: int, head_dim: int, intermediate: int,
              w_std: float = 0.02, couple: bool = True, workers: Optional[int] = None) -> StepCase:
    """Layer l is layer_case(seed * 1000 + l, ...) (its own weights and cache, the same context
    lengths); embeddings ~ N(0, 1) bf16; tokens uniform in [0, vocab)."""
    tokens = stream(seed, TID_TOK).integers(0, vocab, size=batch).astype(np.int32)
    e1 = f32_to_bf16_bits(_normal(seed, TID_E1, (), (vocab, hidden)))
    e2 = f32_to_bf16_bits(_normal(seed, TID_E2, (), (vocab, hidden)))
    layers = [layer_case(seed * 1000 + l, batch=batch, context=context, hidden=hidden, num_q_heads=num_q_heads,
                         num_kv_heads=num_kv_heads, head_dim=head_dim, intermediate=intermediate,
                         w_std=w_std, couple=couple, workers=workers) for l in range(n_layers)]
    return StepCase(seed, tokens, e1, e2, layers)


@dataclass
class HeadCase:
    """Inputs of the shared output head: both flows' final residual rows, the final norm gain,
    the shared vocabulary matrix and uniform noise for a Gumbel-max draw."""
    seed: int
    eps: float
    x: np.ndarray       # float32 [F][B][hidden]
    gain: np.ndarray    # float32 [hidden]
    w_out: np.ndarray   # uint16 [vocab][hidden]
    noise: np.ndarray   # float32 [B][vocab], uniform in (0, 1)


def head_case(seed: int, n_flows: int, batch: int, hidden: int, vocab: int, w_std: float = 0.02,
              x_std: float = 1.0, eps: float = 1e-5, workers: Optional[int] = None) -> HeadCase:
    """Residual rows ~ N(0, x_std), gain ~ U(0.9, 1.1), W_out ~ N(0, w_std) bf16, noise ~
    U(0, 1) with exact 0 moved to the smallest positive fp32 (so every log is finite)."""
    workers = workers or _workers()
    x = _normal(seed, TID_HX, (), (n_flows, batch, hidden), x_std)
    g = _uniform(seed, TID_HG, (), (hidden,), 0.9, 1.1)
    w = _bf16_matrix(seed, TID_WOUT, vocab, hidden, w_std, workers)
    u = stream(seed, TID_NOISE).random((batch, vocab), dtype=np.float32)
    u[u <= 0] = np.float32(np.finfo(np.float32).tiny)
    return HeadCase(seed, eps, x, g, w, u)


@dataclass
class MoeCase:
    """Inputs of the mixture-of-experts MLP block: residual rows of both flows, the norm gain,
    the shared router, every expert's gate/up and down matrices and the coupling vectors."""
    seed: int
    eps: float
    x: np.ndarray          # float32 [2][B][hidden]
    gain: np.ndarray       # float32 [hidden]
    w_router: np.ndarray   # uint16 [E][hidden]
    w_gate_up: np.ndarray  # uint16 [E][2I][hidden]: gate rows, then up rows
    w_down: np.ndarray     # uint16 [E][hidden][I]
    b: Optional[np.ndarray]  # float32 [I] or None
    c: Optional[np.ndarray]  # float32 [hidden] or None


def moe_case(seed: int, batch: int, hidden: int, num_experts: int, intermediate: int,
             w_std: float = 0.02, router_std: float = 0.02, couple: bool = True, eps: float = 1e-5,
             workers: Optional[int] = None) -> MoeCase:
    """Rows ~ N(0, 1), gain ~ U(0.9, 1.1), expert matrices ~ N(0, w_std) and the router ~
    N(0, router_std) in bf16 (expert e's matrices from sub-streams keyed by e), coupling
    vectors ~ U(-1, 1)."""
    workers = workers or _workers()
    E, I = num_experts, intermediate
    x = _normal(seed, TID_MX, (), (2, batch, hidden))
    g = _uniform(seed, TID_MG, (), (hidden,), 0.9, 1.1)
    wr = _bf16_matrix(seed, TID_WR, E, hidden, router_std, workers)
    wgu = np.stack([_bf16_matrix(seed * 1000 + e, TID_WEGU, 2 * I, hidden, w_std, workers) for e in range(E)])
    wd = np.stack([_bf16_matrix(seed * 1000 + e, TID_WED, hidden, I, w_std, workers) for e in range(E)])
    b = _uniform(seed, TID_MB, (), (I,), -1.0, 1.0) if couple else None
    c = _uniform(seed, TID_MC, (), (hidden,), -1.0, 1.0) if couple else None
    return MoeCase(seed, eps, x, g, wr, wgu, wd, b, c)


def config_attention(idx: int, workers: Optional[int] = None, **over) -> AttnCase:
    """The four attention workloads (seed 101 * idx)."""
    seed = 101 * idx
    if idx == 1:
        kw = dict(batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64,
                  context_lens=np.full(1, 512, np.int32), dtype="f32", paged=False)
    elif idx == 2:
        kw = dict(batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
                  context_lens=np.full(16, 4096, np.int32), dtype="bf16", paged=False)
    elif idx == 3:
        kw = dict(batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                  context_lens=ragged_lengths(seed, 64, 1024, 16384), dtype="bf16", paged=True,
                  block_size=16, num_blocks=70000)
    elif idx == 4:
        kw = dict(batch=8, num_q_heads=64, num_kv_heads=8, head_dim=128,
                  context_lens=np.full(8, 131072, np.int32), dtype="bf16", paged=True,
                  block_size=16, num_blocks=65536)
    else:
        raise ValueError(idx)
    kw.update(over)
    return attention_case(seed, workers=workers, **kw)


def config_layer(workers: Optional[int] = None, **over) -> LayerCase:
    """The one-layer workload: B 32, context 8192, hidden 4096, 32/8 heads x 128, MLP 14336."""
    kw = dict(batch=32, context=8192, hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128,
              intermediate=14336, num_blocks=16384)
    kw.update(over)
    return layer_case(505, workers=workers, **kw)
