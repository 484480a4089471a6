"""GPU checks of the measurement helpers (dfx_copy_bytes, dfx_fill_bytes, dfx_read_bytes): the
copy and fill write exactly the bytes asked for, and the read touches every 16-byte word
exactly once (the XOR of what the threads report equals the XOR of the buffer's words)."""
import numpy as np
import pytest
import torch

import dual_flow_shared_amd as dfx
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 3 * 4096 + 48, (1 << 22) + 4096 * 5 + 16 * 7, 64 << 20])
def test_read_touches_every_word_once(nbytes):
    words = np.random.default_rng(nbytes).integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = dev(words.view(np.int32))
    sink = torch.zeros(4096 * 256, dtype=torch.int32, device="cuda")
    dfx.read_bytes(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_copy_and_fill_write_exactly_their_bytes():
    n = (1 << 20) + 48
    src = dev(np.random.default_rng(1).integers(-1 << 31, 1 << 31, n // 4 + 8, dtype=np.int64).astype(np.int32))
    dst = torch.full((n // 4 + 8,), -7, dtype=torch.int32, device="cuda")
    dfx.copy_bytes(dst[: n // 4], src[: n // 4])
    torch.cuda.synchronize()
    assert torch.equal(dst[: n // 4], src[: n // 4]) and bool((dst[n // 4:] == -7).all())
    dfx.fill_bytes(dst[: n // 4], 0x01020304)
    torch.cuda.synchronize()
    assert bool((dst[: n // 4] == 0x01020304).all()) and bool((dst[n // 4:] == -7).all())
