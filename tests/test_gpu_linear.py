"""GPU parity of the grouped linear, RMSNorm, SwiGLU coupling and primary K/V append."""
import numpy as np
import pytest
import torch

import dfx_inputs as gen
import dual_flow_shared_amd as dfx
from gpu_util import bf16_decisions_agree, cache_of, dev, host_bits, max_err
from oracle.cache import kv_append
from oracle.linear import grouped_linear, rmsnorm, swiglu_couple

pytestmark = pytest.mark.gpu

LIN = [
    # (F, rows, K, N)
    (2, 32, 4096, 6144),
    (2, 32, 4096, 4096),
    (2, 32, 14336, 4096),
    (1, 32, 4096, 4096),
    (2, 3, 96, 48),
    (1, 1, 32, 16),
    (2, 40, 256, 128),      # rows of one flow span two row groups
    (1, 100, 512, 64),
    (2, 17, 4128, 272),     # ragged K splits (129 k-steps) and an odd number of 16-column groups
]


@pytest.mark.parametrize("shape", LIN, ids=[str(s) for s in LIN])
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_grouped_linear(shape, x_dtype):
    F, rows, K, N = shape
    c = gen.linear_case(700 + K + N + rows, F, rows, K, N, x_dtype=x_dtype, with_couple=True,
                        with_residual=True)
    x, w = dev(c.x), dev(c.w)
    y = dfx.grouped_linear(x, w)
    yc = dfx.grouped_linear(x, w, couple=dev(c.couple), residual=dev(c.residual))
    wp = dfx.pack_weight(w)
    yp = dfx.grouped_linear(x, wp, packed=True, couple=dev(c.couple), residual=dev(c.residual))
    torch.cuda.synchronize()
    assert max_err(y.cpu().numpy(), grouped_linear(c.x, c.w)) < 2e-3
    want = grouped_linear(c.x, c.w, couple=c.couple, residual=c.residual)
    assert max_err(yc.cpu().numpy(), want) < 2e-3
    assert torch.equal(yp, yc)            # same arithmetic, only the weight order differs


def test_pack_weight_is_the_fragment_permutation():
    rng = np.random.default_rng(5)
    N, K = 48, 96
    w = rng.integers(0, 65535, size=(N, K), dtype=np.uint16)
    got = host_bits(dfx.pack_weight(dev(w)))
    # packed[s][t][lane = n + 16 j][v] = w[16 t + n][32 s + 8 j + v]
    want = w.reshape(N // 16, 16, K // 32, 4, 8).transpose(2, 0, 3, 1, 4).reshape(N, K)
    assert np.array_equal(got, want)


def test_grouped_linear_flow0_independent_of_flows_and_rows():
    c = gen.linear_case(711, 2, 32, 4096, 4096)
    x, w = dev(c.x), dev(c.w)
    y2 = dfx.grouped_linear(x, w)
    y1 = dfx.grouped_linear(x[:1].contiguous(), w)
    y0 = dfx.grouped_linear(x[:1, :5].contiguous(), w)
    torch.cuda.synchronize()
    assert torch.equal(y2[0], y1[0]) and torch.equal(y1[0, :5], y0[0])
    again = dfx.grouped_linear(x, w)
    torch.cuda.synchronize()
    assert torch.equal(again, y2)


def test_grouped_linear_bf16_out_and_in_place_residual():
    c = gen.linear_case(712, 2, 32, 1024, 512, with_residual=True)
    x, w = dev(c.x), dev(c.w)
    yb = dfx.grouped_linear(x, w, y_dtype=torch.bfloat16)
    res = dev(c.residual)
    out = dfx.grouped_linear(x, w, residual=res, out=res)     # in place
    torch.cuda.synchronize()
    # recursive fp32 summation of K products errs by at most K * 2^-24 * sum_k |x_k w_k|
    from oracle.numerics import widen
    scale = np.abs(widen(c.x)) @ np.abs(widen(c.w)).T
    bf16_decisions_agree(host_bits(yb), grouped_linear(c.x, c.w), rel=1024 * 2.0 ** -24, scale=scale)
    assert out.data_ptr() == res.data_ptr()
    assert max_err(res.cpu().numpy(), grouped_linear(c.x, c.w, residual=c.residual)) < 2e-3


@pytest.mark.parametrize("rows,dim", [(64, 4096), (3, 256), (1, 16384)])
def test_rmsnorm(rows, dim):
    rng = np.random.default_rng(rows + dim)
    x = (rng.standard_normal((rows, dim)) * 2).astype(np.float32)
    g = rng.uniform(0.9, 1.1, dim).astype(np.float32)
    y = dfx.rmsnorm(dev(x), dev(g), 1e-5)
    torch.cuda.synchronize()
    frac = bf16_decisions_agree(host_bits(y), _unrounded_rmsnorm(x, g, 1e-5))
    assert frac > 0.99
    assert np.array_equal(host_bits(y)[:, :0], np.zeros((rows, 0), np.uint16))


def _unrounded_rmsnorm(x, g, eps):
    X = x.astype(np.float64)
    return X / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + eps) * g.astype(np.float64)


@pytest.mark.parametrize("flows", [1, 2])
def test_swiglu_couple(flows):
    rng = np.random.default_rng(3 + flows)
    I = 14336
    gu = (rng.standard_normal((flows, 32, 2 * I)) * 2).astype(np.float32)
    b = rng.uniform(-1, 1, I).astype(np.float32)
    y = dfx.swiglu_couple(dev(gu), dev(b))
    torch.cuda.synchronize()
    G = gu.astype(np.float64)
    inter = G[..., :I] / (1 + np.exp(-G[..., :I])) * G[..., I:]
    scale = np.abs(inter).copy()
    if flows == 2:
        scale[1] = np.abs(inter[1]) + np.abs(b * inter[0])   # the coupled sum may cancel
        inter[1] = inter[1] + b * inter[0]
    bf16_decisions_agree(host_bits(y), inter, rel=1e-5, scale=scale)
    # the oracle routine rounds the same values
    assert np.mean(host_bits(y) == _bits(swiglu_couple(gu, b))) > 0.99


def _bits(v):
    from oracle.numerics import bf16_bits
    return bf16_bits(v)


@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("paged", [True, False])
def test_kv_append_bit_exact(src, paged):
    case = gen.attention_case(720, 4, 32, 8, 128, [5, 16, 40, 1], dtype="bf16", paged=paged,
                              capacity=64)
    rng = np.random.default_rng(9)
    pos = np.array([5, 16, 63, 0], np.int32)
    kn = rng.standard_normal((4, 2 * 8 * 128)).astype(np.float32)  # row stride 2048: a wider source row
    vn = rng.standard_normal((4, 2 * 8 * 128)).astype(np.float32)
    if src == "bf16":
        kn, vn = gen.f32_to_bf16_bits(kn), gen.f32_to_bf16_bits(vn)
    cache = cache_of(case)
    kt, vt = dev(kn), dev(vn)
    dfx.kv_append_primary(cache, dev(pos), kt[:, :1024], vt[:, :1024])
    dfx.kv_append_primary(cache, dev(pos), kt[:, :1024], vt[:, :1024])   # idempotent
    torch.cuda.synchronize()
    wk, wv = kv_append(case.k_pool, case.v_pool, case.block_table, pos, kn[:, :1024], vn[:, :1024])
    assert np.array_equal(host_bits(cache.k), wk) and np.array_equal(host_bits(cache.v), wv)
