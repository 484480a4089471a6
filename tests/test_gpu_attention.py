"""GPU parity of dfx_decode_attn against the fp64 oracle, and the properties the pages fix.

Tolerances: max-abs 1e-5 for fp32 inputs, 2e-3 for bf16 inputs (outputs are fp32).
Bit-exact: Q2 = Q1 gives O2 = O1; O1 does not change when the auxiliary flow is added;
the same logical cache through a contiguous, identity-paged or permuted-paged layout;
repeated calls (determinism); the pool is only read.
"""
import hashlib

import numpy as np
import pytest
import torch

import dfx_inputs as gen
from gpu_util import cache_of, dev, lse_err, max_err, run_attn
from oracle.attention import decode_attention

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


def oracle(case, q2=True, a=True, batches=None, q1=None, q2v=None):
    return decode_attention(case.q1 if q1 is None else q1,
                            (case.q2 if q2v is None else q2v) if q2 else None,
                            case.a if (a and q2) else None, case.a_head_stride, case.k_pool,
                            case.v_pool, case.block_table, case.context_lens, batches=batches)


def check(case, got, want, rows=None):
    tol = TOL[case.dtype]
    o1, o2, lse = got
    w1, w2, wl = want
    e1 = max_err(o1, w1, rows)
    e2 = max_err(o2, w2, rows) if w2 is not None else 0.0
    el = lse_err(lse[:, rows] if rows is not None else lse, wl[:, rows] if rows is not None else wl)
    assert e1 < tol and e2 < tol, (e1, e2)
    assert el < tol, el
    return e1, e2


def test_fp32_single_layer_workload():
    case = gen.config_attention(1)
    check(case, run_attn(case), oracle(case))


SHAPES = [
    # (B, Hq, Hkv, D, ctx list, paged, dtype)
    (2, 8, 8, 64, [1, 2], True, "bf16"),
    (3, 8, 2, 128, [15, 16, 17], True, "bf16"),
    (2, 16, 2, 128, [33, 100], True, "bf16"),
    (2, 32, 8, 128, [129, 1000], False, "bf16"),
    (1, 8, 1, 64, [777], True, "bf16"),
    (2, 4, 4, 64, [5, 300], True, "f32"),
    (2, 64, 4, 128, [200, 31], True, "bf16"),   # 16 query heads per KV head: 32 rows, VALU path
    (3, 12, 4, 128, [0, 50, 2], True, "bf16"),  # empty context
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(i) for i in range(len(SHAPES))])
@pytest.mark.parametrize("per_head", [False, True])
def test_small_shapes(shape, per_head):
    B, Hq, Hkv, D, ctx, paged, dt = shape
    case = gen.attention_case(500 + sum(ctx) + B, B, Hq, Hkv, D, ctx, dtype=dt, paged=paged,
                              a_per_head=per_head)
    check(case, run_attn(case), oracle(case))
    # primary-only call
    o1, o2, lse = run_attn(case, q2=False)
    w1, _, wl = oracle(case, q2=False)
    assert o2 is None and max_err(o1, w1) < TOL[dt]


@pytest.mark.parametrize("D,paged,q_dtype", [(128, True, "bf16"), (64, True, "bf16"), (128, False, "bf16"),
                                            (64, False, "f32")])
def test_large_batch_whole_row_k_tiles(D, paged, q_dtype):
    """At 512 or more (sequence, KV head) pairs the kernel stages K tiles through LDS as whole
    rows: ragged lengths with empty, one-token and tail-tile sequences, both layouts."""
    B, Hkv = 128, 4
    ctx = np.random.default_rng(D + paged).integers(1, 300, B).astype(np.int32)
    ctx[:4] = [0, 1, 31, 33]
    case = gen.attention_case(620 + D + paged, B, 8, Hkv, D, ctx, dtype="bf16", paged=paged)
    if q_dtype == "f32":  # fp32 queries (the same values) against the bf16 cache
        case.q1, case.q2 = gen.bf16_bits_to_f32(case.q1), gen.bf16_bits_to_f32(case.q2)
    check(case, run_attn(case), oracle(case))
    check(case, run_attn(case, num_splits=3), oracle(case))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 32])
def test_split_counts(splits):
    case = gen.attention_case(601, 3, 32, 8, 128, [4096, 1500, 3001], dtype="bf16", paged=True)
    check(case, run_attn(case, num_splits=splits), oracle(case))


def test_shared_workspace_across_shapes_and_splits():
    """One workspace serves calls of changing shape and split count: each result equals a
    fresh workspace's bit for bit (split partials are fully written before they are read)."""
    import dual_flow_shared_amd as dfx
    ws = dfx.Workspace()
    cases = [(gen.attention_case(611, 3, 32, 8, 128, [4096, 1500, 3001], dtype="bf16", paged=True), 7),
             (gen.attention_case(612, 9, 16, 8, 64, [700] * 9, dtype="bf16", paged=True), 2),
             (gen.attention_case(613, 2, 32, 4, 128, [2500, 600], dtype="bf16"), 5),
             (gen.attention_case(611, 3, 32, 8, 128, [4096, 1500, 3001], dtype="bf16", paged=True), 3)]
    for _ in range(2):
        for case, splits in cases:
            cache, ctx = cache_of(case), dev(case.context_lens)
            args = (dev(case.q1), dev(case.q2), dev(case.a))
            kw = dict(cache=cache, context_lens=ctx, max_context=int(case.context_lens.max()), num_splits=splits)
            got = dfx.decode_attn(*args, workspace=ws, **kw)
            fresh = dfx.decode_attn(*args, workspace=dfx.Workspace(), **kw)
            torch.cuda.synchronize()
            for g, f in zip(got, fresh):
                assert torch.equal(g, f)


def test_contiguous_batch16_context4096():
    case = gen.config_attention(2)
    check(case, run_attn(case), oracle(case))


def test_q2_equal_q1_bit_identical():
    case = gen.attention_case(602, 2, 32, 8, 128, [900, 2048], dtype="bf16")
    o1, o2, _ = run_attn(case, q2v=case.q1, a=False)
    assert np.array_equal(o1, o2)
    cache = cache_of(case)
    ctx = dev(case.context_lens)
    q1 = dev(case.q1)
    import dual_flow_shared_amd as dfx
    z = torch.zeros_like(q1)
    ones = torch.ones(128, dtype=torch.float32, device="cuda")
    p1, p2, _ = dfx.decode_attn(q1, z, ones, cache=cache, context_lens=ctx, max_context=2048)
    zeros = torch.zeros(128, dtype=torch.float32, device="cuda")
    r1, r2, _ = dfx.decode_attn(q1, q1, zeros, cache=cache, context_lens=ctx, max_context=2048)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(r1, r2) and torch.equal(p1, r1)


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_primary_unchanged_by_aux(splits):
    case = gen.attention_case(603, 4, 32, 8, 128, [3000, 17, 1024, 2500], dtype="bf16")
    d1, d2, dl = run_attn(case, num_splits=splits)
    s1, s2, sl = run_attn(case, q2=False, num_splits=splits)
    assert s2 is None and np.array_equal(d1, s1) and np.array_equal(dl[0], sl[0])


def test_dual_equals_single_with_materialized_q2():
    case = gen.attention_case(604, 2, 32, 8, 128, [2000, 700], dtype="bf16")
    _, o2, _ = run_attn(case)
    from oracle.numerics import widen
    q2 = (widen(case.q2) + widen(case.a)[None, None, :] * widen(case.q1)).astype(np.float32)
    s1, _, _ = run_attn(case, q1=q2, q2=False)
    assert max_err(o2, s1) < 2e-3


def test_layouts_bit_identical_and_cache_read_only():
    kw = dict(batch=3, num_q_heads=32, num_kv_heads=8, head_dim=128, context_lens=[1000, 64, 1777],
              dtype="bf16")
    paged = gen.attention_case(605, paged=True, **kw)
    contig = gen.attention_case(605, paged=False, **kw)
    ident = gen.attention_case(605, paged=True, **kw)
    # identity table over a packed pool holding the same logical rows
    nblk = [-(-n // 16) for n in kw["context_lens"]]
    width = max(nblk)
    table = np.zeros((3, width), np.int32)
    pool_k = np.full((sum(nblk) + 1, 8, 16, 128), gen.BF16_QNAN, np.uint16)
    pool_v = pool_k.copy()
    off = 0
    for b, k in enumerate(nblk):
        table[b, :k] = np.arange(off, off + k)
        table[b, k:] = sum(nblk)
        pool_k[off:off + k] = paged.k_pool[paged.block_table[b, :k]]
        pool_v[off:off + k] = paged.v_pool[paged.block_table[b, :k]]
        off += k
    ident.block_table, ident.k_pool, ident.v_pool = table, pool_k, pool_v
    cache = cache_of(paged)
    before = hashlib.sha256(cache.k.view(torch.int16).cpu().numpy().tobytes()
                            + cache.v.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
    a = run_attn(paged, cache=cache)
    a2 = run_attn(paged, cache=cache)
    after = hashlib.sha256(cache.k.view(torch.int16).cpu().numpy().tobytes()
                           + cache.v.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
    assert before == after
    b = run_attn(contig, max_context=1777)
    c = run_attn(ident)
    for x, y, z, w in zip(a, a2, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z) and np.array_equal(x, w)


@pytest.mark.parametrize("paged,splits", [(True, 0), (True, 3), (False, 2)])
def test_context_lengths_above_max_context_are_clamped(paged, splits):
    """A sequence whose context_lens entry exceeds max_context attends to max_context
    positions (n_b = min(context_lens[b], max_context)); negative entries count as 0."""
    case = gen.attention_case(615, 4, 16, 4, 128, [300, 90, 250, 5], dtype="bf16", paged=paged)
    mc = 200
    lens = np.array([300, 90, 250, -7], np.int32)
    got = run_attn(case, num_splits=splits, max_context=mc, ctx=lens)
    clamped = gen.attention_case(615, 4, 16, 4, 128, [300, 90, 250, 5], dtype="bf16", paged=paged)
    clamped.context_lens = np.minimum(np.maximum(lens, 0), mc).astype(np.int32)
    check(clamped, got, oracle(clamped))


def test_one_token_returns_v_and_constant_v():
    case = gen.attention_case(606, 4, 32, 8, 128, [1, 1, 1, 1], dtype="bf16")
    o1, o2, _ = run_attn(case)
    from oracle.numerics import widen
    for b in range(4):
        blk = case.block_table[b, 0]
        v = widen(case.v_pool[blk, :, 0])                         # [Hkv][D]
        assert np.array_equal(o1[b], np.repeat(v, 4, axis=0)) and np.array_equal(o2[b], np.repeat(v, 4, axis=0))
    case = gen.attention_case(607, 2, 32, 8, 128, [3000, 129], dtype="bf16")
    case.v_pool[:] = 0x3F80                                       # V = 1
    o1, o2, _ = run_attn(case)
    # weights sum to one up to fp32 summation over 3000 terms
    assert max_err(o1, np.ones_like(o1)) < 1e-5 and max_err(o2, np.ones_like(o2)) < 1e-5


@pytest.mark.parametrize("gain", [40.0, 150.0])
@pytest.mark.parametrize("splits", [1, 3, 8])
def test_peaked_softmax_and_far_apart_split_maxima(gain, splits):
    """Queries scaled so that scores spread over tens to hundreds of units: the softmax is
    nearly one-hot, most terms underflow, and the splits' maxima differ by far more than
    exp's range -- the online rescale and the merge must lose nothing. Outputs within the
    bf16 bar. lse, now of magnitude up to ~5 * gain, within the error that the kernel's query
    representation allows: an fp32 query (the auxiliary's, q2_raw + a * q1) is carried as two
    bf16 terms, about 2^-17 relative per element, so a score is off by at most
    2^-16 * scale * sum_d |Q_d K_d| and the lse (a smooth maximum of the scores) by the
    largest such bound over the keys."""
    case = gen.attention_case(640, 2, 8, 2, 128, [1000, 777], dtype="bf16", paged=True)
    for name in ("q1", "q2"):
        q = gen.bf16_bits_to_f32(getattr(case, name)) * np.float32(gain)
        setattr(case, name, gen.f32_to_bf16_bits(q))
    o1, o2, lse = run_attn(case, num_splits=splits)
    w1, w2, wl = oracle(case)
    assert max_err(o1, w1) < 2e-3 and max_err(o2, w2) < 2e-3, (max_err(o1, w1), max_err(o2, w2))
    D, G, bs = case.head_dim, case.num_q_heads // case.num_kv_heads, case.block_size
    q1 = gen.bf16_bits_to_f32(case.q1).astype(np.float64)
    qs = (q1, gen.bf16_bits_to_f32(case.q2).astype(np.float64) + case.a.astype(np.float64) * q1)
    bound = np.empty_like(wl)
    for b, n in enumerate(case.context_lens):
        blocks = case.block_table[b, : -(-n // bs)]
        for h in range(case.num_q_heads):
            k = gen.bf16_bits_to_f32(case.k_pool[blocks, h // G]).reshape(-1, D)[:n].astype(np.float64)
            for f in range(2):
                bound[f, b, h] = 2.0 ** -16 / np.sqrt(D) * (np.abs(k) @ np.abs(qs[f][b, h])).max()
    err = np.abs(lse - wl)
    assert np.all(err <= 1e-4 + bound), float((err / (1e-4 + bound)).max())


def test_ragged_paged_full_size_sampled():
    """The ragged 64-sequence workload: the shortest and the longest sequence and ten more
    seeded ones against the oracle."""
    case = gen.config_attention(3)
    n = case.context_lens
    rows = sorted({int(np.argmin(n)), int(np.argmax(n))} | set(int(r) for r in np.random.default_rng(3).choice(64, 10, replace=False)))
    print("ragged workload: sequences", rows, "contexts", [int(n[r]) for r in rows], flush=True)
    got = run_attn(case)
    want = oracle(case, batches=rows)
    check(case, got, want, rows=rows)
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))


def test_largest_batch_sampled():
    """65535 sequences (the grid's largest y extent) of 0-19 tokens: sampled sequences against
    the oracle, with the planner's single split and with two splits and the merge."""
    B = 65535
    ctx = np.random.default_rng(17).integers(0, 20, B).astype(np.int32)
    ctx[[0, 1]] = [0, 19]
    case = gen.attention_case(905, B, 8, 1, 64, ctx, dtype="bf16", paged=True)
    rows = [0, 1, 2, 32767, B - 1]
    want = oracle(case, batches=rows)
    for splits in (0, 2):
        got = run_attn(case, num_splits=splits)
        check(case, got, want, rows=rows)
        assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))


def test_long_context_reduced_twin():
    case = gen.attention_case(404, 8, 64, 8, 128, np.full(8, 8192, np.int32), dtype="bf16",
                              paged=True, num_blocks=8 * 512 + 9)
    check(case, run_attn(case), oracle(case))


def test_long_context_full_size_all_sequences():
    """The 131072-token workload, every sequence of the batch against the oracle."""
    case = gen.config_attention(4)
    got = run_attn(case)
    check(case, got, oracle(case))
