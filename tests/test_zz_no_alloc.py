"""The allocation-free decode attention (dfx_decode_attn_noalloc) against dfx_decode_attn, through
the C ABI: the same plan and kernels, so the same bits, on two calls in a row, the second with
a smaller input (the shared scratch array keeps the first call's partials)."""
import ctypes

import numpy as np
import pytest
import torch

import dfx_inputs as gen
from dual_flow_shared_amd import _abi
from gpu_util import cache_of, dev

pytestmark = pytest.mark.gpu


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def both(case, splits):
    """dfx_decode_attn with a caller workspace and dfx_decode_attn_noalloc, same arguments."""
    lib = _abi.lib()
    cache = cache_of(case)
    st = cache.struct()
    B, Hq, D = case.batch, case.num_q_heads, case.head_dim
    mc = int(case.context_lens.max())
    q1, q2, a, ctx = dev(case.q1), dev(case.q2), dev(case.a), dev(case.context_lens)
    qdt = _abi.DFX_BF16 if case.q1.dtype == np.uint16 else _abi.DFX_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    n = ctypes.c_size_t()
    assert lib.dfx_decode_attn_workspace_size(B, Hq, 2, ctypes.byref(st), mc, splits, ctypes.byref(n)) == 0
    assert n.value > 0, "the case must use split partials"
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    for noalloc in (False, True):
        o1 = torch.full((B, Hq, D), float("nan"), device="cuda")
        o2 = torch.full((B, Hq, D), float("nan"), device="cuda")
        lse = torch.full((2, B, Hq), float("nan"), device="cuda")
        if noalloc:
            r = lib.dfx_decode_attn_noalloc(ctypes.byref(st), ptr(ctx), B, mc, Hq, qdt, ptr(q1), ptr(q2), 0, ptr(a),
                                            case.a_head_stride, 0.0, ptr(o1), ptr(o2), ptr(lse), splits, stream)
        else:
            r = lib.dfx_decode_attn(ctypes.byref(st), ptr(ctx), B, mc, Hq, qdt, ptr(q1), ptr(q2), 0, ptr(a),
                                    case.a_head_stride, 0.0, ptr(o1), ptr(o2), ptr(lse), splits, ptr(ws), n.value,
                                    stream)
        assert r == 0, lib.dfx_last_error().decode()
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (o1, o2, lse)])
    return outs


def test_noalloc_attention_equals_workspace_attention_on_two_calls():
    # first call: 5 sequences of ragged length over a paged cache, 6 splits (the scratch is
    # filled with partials of 6 x 2 x 5 x 32 rows)
    big = gen.attention_case(2101, 5, 32, 8, 128, [3000, 1, 4096, 777, 2500], dtype="bf16", paged=True)
    # second call: fewer sequences, fewer splits, fp32 queries and cache on the vector kernel:
    # it reads only what it writes, whatever the first call left in the array
    small = gen.attention_case(2102, 2, 8, 2, 64, [300, 45], dtype="f32", paged=True)
    for case, splits in ((big, 6), (small, 3)):
        print(f"noalloc attention: batch {case.batch}, {case.num_q_heads}/{case.num_kv_heads} x {case.head_dim}, "
              f"{case.dtype}, {splits} splits", flush=True)
        ref, got = both(case, splits)
        for r, g in zip(ref, got):
            assert np.all(np.isfinite(r))
            assert np.array_equal(r.view(np.uint32), g.view(np.uint32))
