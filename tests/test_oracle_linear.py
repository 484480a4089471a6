"""Pins for the oracle's grouped linear, RMSNorm and SwiGLU coupling (CPU only)."""
import numpy as np
import torch
import torch.nn.functional as Fn

import dfx_inputs as gen
from oracle.linear import grouped_linear, rmsnorm, swiglu_couple
from oracle.numerics import round_bf16


def t64(bits_or_f32):
    a = np.asarray(bits_or_f32)
    if a.dtype == np.uint16:
        a = gen.bf16_bits_to_f32(a)
    return torch.from_numpy(a.astype(np.float64))


def test_grouped_linear_matches_library_per_flow():
    c = gen.linear_case(1, 2, 5, 96, 40, x_dtype="bf16")
    y = grouped_linear(c.x, c.w)
    for f in range(2):
        ref = Fn.linear(t64(c.x[f]), t64(c.w)).numpy()
        assert np.max(np.abs(y[f] - ref)) < 1e-12


def test_fp32_rows_are_rounded_to_bf16_first():
    c = gen.linear_case(2, 2, 3, 64, 24, x_dtype="f32")
    y = grouped_linear(c.x, c.w)
    xb = torch.from_numpy(c.x).to(torch.bfloat16).to(torch.float64)   # library RNE cast
    ref = Fn.linear(xb, t64(c.w)).numpy()
    assert np.max(np.abs(y - ref)) < 1e-12


def test_flows_are_independent_and_share_weights():
    c = gen.linear_case(3, 2, 4, 64, 32)
    y2 = grouped_linear(c.x, c.w)
    y1 = grouped_linear(c.x[:1], c.w)
    assert np.array_equal(y2[0], y1[0])
    swapped = grouped_linear(c.x[::-1].copy(), c.w)
    assert np.array_equal(swapped[0], y2[1]) and np.array_equal(swapped[1], y2[0])


def test_couple_and_residual():
    c = gen.linear_case(4, 2, 3, 64, 32, with_couple=True, with_residual=True)
    x = np.stack([c.x[0], c.x[0]])                       # aux rows equal primary rows
    y0 = grouped_linear(x, c.w)
    # couple = -1 cancels the aux row exactly; couple = 0 leaves it equal to the primary
    assert np.all(grouped_linear(x, c.w, couple=np.full(32, -1, np.float32))[1] == 0)
    assert np.array_equal(grouped_linear(x, c.w, couple=np.zeros(32, np.float32))[1], y0[0])
    y = grouped_linear(c.x, c.w, couple=c.couple, residual=c.residual)
    base = [Fn.linear(t64(c.x[f]), t64(c.w)).numpy() for f in range(2)]
    assert np.max(np.abs(y[0] - (c.residual[0] + base[0]))) < 1e-12
    # the aux row gets couple * (primary product), taken before the residual add
    assert np.max(np.abs(y[1] - (c.residual[1] + base[1] + c.couple * base[0]))) < 1e-12
    yb = grouped_linear(c.x, c.w, y_bf16=True)
    assert yb.dtype == np.uint16


def test_rmsnorm_matches_library():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 256)) * 3
    g = rng.uniform(0.9, 1.1, 256)
    ours = rmsnorm(x, g, 1e-5)
    ref = Fn.rms_norm(torch.from_numpy(x), (256,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    # one bf16 rounding of the library value; the two fp64 values may differ in the last
    # bits, so an element next to a rounding midpoint may land one bf16 step away
    same = ours == round_bf16(ref)
    assert same.mean() > 0.999
    assert np.all(np.abs(ours - ref)[~same] <= np.abs(ref)[~same] * 2.0 ** -7)


def test_swiglu_matches_library_and_couples():
    rng = np.random.default_rng(6)
    gu = rng.standard_normal((2, 3, 2 * 48)) * 2
    b = rng.uniform(-1, 1, 48)
    ours = swiglu_couple(gu, b)
    t = torch.from_numpy(gu)
    inter = Fn.silu(t[..., :48]) * t[..., 48:]
    ref = inter.numpy().copy()
    same = ours[0] == round_bf16(ref[0])
    assert same.mean() > 0.99
    assert np.all(np.abs(ours[0] - ref[0])[~same] <= np.abs(ref[0])[~same] * 2.0 ** -7)
    same = np.stack([gu[0], gu[0]])
    assert np.all(swiglu_couple(same, np.full(48, -1.0))[1] == 0)
    assert np.array_equal(swiglu_couple(same, np.zeros(48))[1], swiglu_couple(same, np.zeros(48))[0])
    assert np.array_equal(swiglu_couple(gu[:1], b)[0], ours[0])
