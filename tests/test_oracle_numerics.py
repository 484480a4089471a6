"""Pins for the oracle's exact widening and direct fp64 -> bf16 rounding."""
import os

import numpy as np
import torch

from oracle.numerics import bf16_bits, round_bf16, widen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne_cases.txt")


def _cases():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        v, bits = line.split()[:2]
        out.append((float.fromhex(v), int(bits, 16)))
    return out


def test_golden_rounding_table():
    cases = _cases()
    assert len(cases) >= 12
    vals = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases], dtype=np.uint16)
    got = bf16_bits(vals)
    bad = [(hex(float(v)), hex(int(g)), hex(int(w))) for v, g, w in zip(vals, got, want) if g != w]
    assert not bad, bad


def test_matches_torch_cast_on_fp32_inputs():
    # torch's float32 -> bfloat16 cast is round-to-nearest-even; on fp32-exact inputs a
    # direct fp64 rounding must agree with it bit for bit (including subnormals and huge values)
    rng = np.random.default_rng(7)
    parts = [rng.standard_normal(200000).astype(np.float32),
             (rng.standard_normal(20000) * 1e37).astype(np.float32),
             (rng.standard_normal(20000) * 1e-39).astype(np.float32),
             rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32)]
    x = np.concatenate(parts)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_widen_exact():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    want = np.array([1.0, -2.0, np.inf, 2.0 ** -133, -0.0, 3.140625])
    got = widen(bits)
    assert np.array_equal(got, want)
    assert np.signbit(got[4])
    assert widen(np.float32(0.1)).item() == float(np.float32(0.1))


def test_round_is_idempotent_and_nan_preserving():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10000) * 10.0
    r = round_bf16(x)
    assert np.array_equal(round_bf16(r), r)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)
    assert np.isnan(round_bf16(np.array([np.nan]))[0])
    assert bf16_bits(np.array([np.nan]))[0] == 0x7FC0
