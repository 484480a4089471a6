"""Pins for the oracle's primary-only K/V append (CPU only): hand-computed slots."""
import numpy as np
import torch

from oracle.cache import kv_append


def test_append_addresses_and_rounding():
    nb, Hkv, bs, D = 9, 2, 4, 8
    k = np.full((nb, Hkv, bs, D), 0x7FC0, np.uint16)
    v = k.copy()
    table = np.array([[5, 2, 8], [0, 7, 8]], np.int32)
    pos = np.array([5, 0])                      # seq 0: block table[0][1] = 2, slot 1; seq 1: block 0, slot 0
    rng = np.random.default_rng(1)
    kn = rng.standard_normal((2, Hkv * D)).astype(np.float32)
    vn = rng.standard_normal((2, Hkv * D)).astype(np.float32)
    kp, vp = kv_append(k, v, table, pos, kn, vn)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kp[2, :, 1], bf(kn[0]).reshape(Hkv, D))
    assert np.array_equal(vp[0, :, 0], bf(vn[1]).reshape(Hkv, D))
    changed = np.argwhere(np.any(kp != k, axis=-1))
    assert sorted(map(tuple, changed)) == [(0, 0, 0), (0, 1, 0), (2, 0, 1), (2, 1, 1)]
    assert np.array_equal(kp[[1, 3, 4, 5, 6, 7, 8]], k[[1, 3, 4, 5, 6, 7, 8]])


def test_append_contiguous_and_bf16_sources_verbatim():
    k = np.zeros((3, 1, 6, 4), np.uint16)
    src = np.arange(3 * 4, dtype=np.uint16).reshape(3, 4) + 0x3F00
    kp, vp = kv_append(k, k.copy(), None, np.array([5, 0, 2]), src, src)
    assert np.array_equal(kp[0, 0, 5], src[0]) and np.array_equal(kp[1, 0, 0], src[1])
    assert np.array_equal(kp[2, 0, 2], src[2]) and np.count_nonzero(kp) == 12
