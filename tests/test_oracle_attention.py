"""Pins for the oracle's dual-query decode attention (CPU only).

Each check compares the oracle with something other than itself: scalar brute
force, torch's scaled_dot_product_attention (a library routine), identities
that follow from the definition (Q2 = Q1 gives O2 = O1; a constant coupling
vector is a temperature; one cached token returns its value row), closed forms
(identical keys give the mean of V), and LSE algebra over a partition of the
context. K/V for the library pins come straight from the input generator's
logical per-(sequence, KV head) streams, not through the pool and table.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import dfx_inputs as gen
from oracle.attention import brute_force, decode_attention
from oracle.numerics import widen


def run(case, q1=None, q2="case", a="case", stride=None, **kw):
    q1 = case.q1 if q1 is None else q1
    q2 = case.q2 if isinstance(q2, str) else q2
    a = case.a if isinstance(a, str) else a
    stride = case.a_head_stride if stride is None else stride
    return decode_attention(q1, q2, a, stride, case.k_pool, case.v_pool, case.block_table,
                            case.context_lens, **kw)


def logical_kv(case, b, g):
    """The generator's own rows for (b, g) -- what the table-gathered cache must hold."""
    n = int(case.context_lens[b])
    k = gen._normal(case.seed, gen.TID_K, (b, g), (n, case.head_dim))
    v = gen._normal(case.seed, gen.TID_V, (b, g), (n, case.head_dim))
    if case.dtype == "bf16":
        k, v = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(k)), gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(v))
    return torch.from_numpy(k.astype(np.float64)), torch.from_numpy(v.astype(np.float64))


def sdpa_ref(case, Q, scale=None):
    """torch SDPA per (b, KV head) with the query heads of that KV head. Q: [B][Hq][D] fp64."""
    B, Hq, D = Q.shape
    G = Hq // case.num_kv_heads
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for g in range(case.num_kv_heads):
            k, v = logical_kv(case, b, g)
            q = torch.from_numpy(np.ascontiguousarray(Q[b, g * G:(g + 1) * G]))
            o = Fn.scaled_dot_product_attention(q[None], k[None], v[None], scale=scale)
            out[b, g * G:(g + 1) * G] = o[0].numpy()
    return out


SMALL = [
    dict(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, context_lens=[17, 33], paged=True),
    dict(batch=3, num_q_heads=8, num_kv_heads=1, head_dim=64, context_lens=[1, 16, 2], paged=True),
    dict(batch=2, num_q_heads=2, num_kv_heads=2, head_dim=128, context_lens=[15, 100], paged=False),
    dict(batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128, context_lens=[47], paged=True),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_brute_force(dtype, idx):
    kw = dict(SMALL[idx])
    case = gen.attention_case(11 + idx, dtype=dtype, a_per_head=bool(idx % 2), **kw)
    o1, o2, lse = run(case)
    bo, blse = brute_force(case.q1, case.q2, case.a, case.a_head_stride, case.k_pool, case.v_pool,
                           case.block_table, case.context_lens)
    assert np.max(np.abs(o1 - bo[0])) < 1e-12
    assert np.max(np.abs(o2 - bo[1])) < 1e-12
    assert np.max(np.abs(lse - blse)) < 1e-12


@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_library_sdpa_per_flow(idx):
    case = gen.attention_case(21 + idx, dtype="bf16", **SMALL[idx])
    # no coupling: each flow is plain attention of its own query over the primary K/V
    o1, o2, _ = run(case, a=None)
    assert np.max(np.abs(o1 - sdpa_ref(case, widen(case.q1)))) < 1e-12
    assert np.max(np.abs(o2 - sdpa_ref(case, widen(case.q2)))) < 1e-12


def test_coupling_constant_vector_is_a_temperature():
    # a = c * ones, q2_raw = 0  =>  Q2 = c * Q1  =>  softmax(c * Q1 K^T / sqrt(D))
    case = gen.attention_case(31, 2, 8, 2, 64, [40, 9], dtype="f32")
    c = float(np.float32(0.37))  # the value the oracle receives
    _, o2, _ = run(case, q2=np.zeros_like(case.q1), a=np.full(64, c, np.float32), stride=0)
    ref = sdpa_ref(case, widen(case.q1), scale=c / math.sqrt(64))
    assert np.max(np.abs(o2 - ref)) < 1e-12


def test_coupling_per_head_vector():
    # per-head constants c_h: each head gets its own temperature; a wrong head index fails
    case = gen.attention_case(32, 1, 8, 2, 64, [50], dtype="f32")
    ch = np.linspace(-0.9, 1.3, 8).astype(np.float32)
    a = np.repeat(ch[:, None], 64, axis=1)
    _, o2, _ = run(case, q2=np.zeros_like(case.q1), a=a, stride=64)
    for h in range(8):
        ref = sdpa_ref(case, widen(case.q1), scale=float(ch[h]) / 8.0)
        assert np.max(np.abs(o2[0, h] - ref[0, h])) < 1e-12


@pytest.mark.parametrize("per_head", [False, True])
def test_coupling_reconstructs_primary(per_head):
    # q2_raw = Q1 * (1 - a)  =>  Q2 = Q1 exactly (up to one fp64 rounding) for ANY a,
    # so O2 = O1; a coupling with a wrong index, sign or broadcast fails this
    case = gen.attention_case(33, 2, 8, 2, 64, [30, 64], dtype="bf16", a_per_head=per_head)
    Q1 = widen(case.q1)
    A = widen(case.a).reshape((1, 1, 64) if not per_head else (1, 8, 64))
    o1, o2, lse = run(case, q2=Q1 * (1.0 - A))
    assert np.max(np.abs(o2 - o1)) < 1e-12
    assert np.max(np.abs(lse[1] - lse[0])) < 1e-12


def test_q2_equal_q1_bit_identical():
    case = gen.attention_case(34, 2, 8, 2, 64, [30, 5], dtype="bf16")
    o1, o2, lse = run(case, q2=case.q1, a=np.zeros(64, np.float32), stride=0)
    assert np.array_equal(o1, o2) and np.array_equal(lse[0], lse[1])
    o1b, o2b, _ = run(case, q2=np.zeros_like(case.q1), a=np.ones(64, np.float32), stride=0)
    assert np.array_equal(o1b, o2b) and np.array_equal(o1b, o1)


def test_aux_does_not_change_primary():
    case = gen.attention_case(35, 2, 8, 2, 64, [30, 5], dtype="bf16")
    o1, o2, lse = run(case)
    p1, none, plse = run(case, q2=None, a=None)
    assert none is None and np.array_equal(o1, p1) and np.array_equal(lse[0], plse[0])


def test_one_token_returns_value_row():
    case = gen.attention_case(36, 3, 8, 4, 128, [1, 1, 1], dtype="bf16")
    o1, o2, lse = run(case)
    for b in range(3):
        for h in range(8):
            _, v = logical_kv(case, b, h // 2)
            assert np.array_equal(o1[b, h], v[0].numpy()) and np.array_equal(o2[b, h], v[0].numpy())


def test_weights_sum_to_one_and_constant_values():
    case = gen.attention_case(37, 2, 8, 2, 64, [300, 77], dtype="bf16")
    _, _, _, W = run(case, return_weights=True)
    for w in W.values():
        assert np.max(np.abs(w.sum(axis=1) - 1.0)) < 1e-12
        assert np.all(w >= 0)
    ones = np.full_like(case.v_pool, 0x3F80)        # V = 1 everywhere
    o1, o2, _ = decode_attention(case.q1, case.q2, case.a, 0, case.k_pool, ones, case.block_table,
                                 case.context_lens)
    assert np.max(np.abs(o1 - 1.0)) < 1e-12 and np.max(np.abs(o2 - 1.0)) < 1e-12


def test_identical_keys_give_mean_value_and_log_n():
    case = gen.attention_case(38, 2, 4, 2, 64, [50, 13], dtype="f32", paged=False)
    kz = np.zeros_like(case.k_pool)                 # K = 0: every score is 0
    o1, o2, lse = decode_attention(case.q1, case.q2, case.a, 0, kz, case.v_pool, None,
                                   case.context_lens)
    for b in range(2):
        n = int(case.context_lens[b])
        for h in range(4):
            mean = case.v_pool[b, h // 2, :n].astype(np.float64).mean(axis=0)
            assert np.max(np.abs(o1[b, h] - mean)) < 1e-12 and np.max(np.abs(o2[b, h] - mean)) < 1e-12
            assert abs(lse[0, b, h] - math.log(n)) < 1e-12


def test_dominant_key():
    # one key aligned with the query at a score gap of >= 60 dominates: O = V of that key
    D = 64
    case = gen.attention_case(39, 1, 1, 1, D, [20], dtype="f32", paged=False)
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros_like(case.k_pool)
    k[0, 0, 7, 0] = 8.0 * 64.0                      # score 64 vs 0 elsewhere
    o1, _, lse = decode_attention(q, None, None, 0, k, case.v_pool, None, case.context_lens)
    # the other 19 weights are e^-64 / (1 + 19 e^-64) < 2e-28 each
    assert np.max(np.abs(o1[0, 0] - case.v_pool[0, 0, 7])) < 1e-24
    assert abs(lse[0, 0, 0] - (64.0 + math.log1p(19 * math.exp(-64.0)))) < 1e-12


def test_lse_partition_merge():
    # attention over [0, n) equals the LSE-weighted merge of attention over any partition
    case = gen.attention_case(40, 2, 8, 2, 64, [97, 97], dtype="bf16", paged=False)
    full1, full2, flse = run(case)
    cuts = [0, 13, 14, 50, 97]
    parts = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        kp, vp = case.k_pool[:, :, lo:hi], case.v_pool[:, :, lo:hi]
        o1, o2, lse = decode_attention(case.q1, case.q2, case.a, 0, kp, vp, None,
                                       np.full(2, hi - lo, np.int32))
        parts.append((np.stack([o1, o2]), lse))
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    O = sum(np.exp(p[1] - L)[..., None] * p[0] for p in parts)
    assert np.max(np.abs(L - flse)) < 1e-12
    assert np.max(np.abs(O - np.stack([full1, full2]))) < 1e-12


def test_paging_invariance():
    # the same logical cache through an identity table, a permuted table, and contiguous
    kw = dict(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, context_lens=[40, 1, 77],
              dtype="bf16")
    a = gen.attention_case(41, paged=True, **kw)
    c = gen.attention_case(41, paged=False, **kw)
    oa = run(a)
    oc = run(c)
    for x, y in zip(oa, oc):
        assert np.array_equal(x, y)


def test_empty_context():
    case = gen.attention_case(42, 2, 4, 2, 64, [0, 5], dtype="bf16")
    o1, o2, lse = run(case)
    assert np.all(o1[0] == 0) and np.all(o2[0] == 0) and np.all(np.isneginf(lse[:, 0]))
    assert np.all(np.isfinite(o1[1]))


def test_poison_never_reaches_outputs():
    case = gen.attention_case(43, 3, 8, 2, 64, [17, 31, 3], dtype="bf16", num_blocks=40)
    o1, o2, lse = run(case)
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(o2)) and np.all(np.isfinite(lse))
