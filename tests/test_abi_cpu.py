"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

from dual_flow_shared_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dfx.h")
FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation first


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dfx_status|int|const char \*)\s*(dfx_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported_and_bound():
    lib = _abi.lib()
    names = declared()
    assert len(names) == 33
    for n in names:
        assert hasattr(lib, n), n
        assert n in _abi.SIGNATURES, n
    assert set(_abi.SIGNATURES) == set(names)
    assert lib.dfx_version() == 100


def kv(dtype=1, heads=8, D=128, bs=16, nb=100, table=FAKE, mb=64):
    s = _abi.KVCacheStruct()
    s.dtype, s.num_kv_heads, s.head_dim, s.block_size, s.num_blocks = dtype, heads, D, bs, nb
    s.k = s.v = FAKE
    s.block_table, s.max_blocks_per_seq, s.reserved = table, mb, 0
    return s


def attn(k, **over):
    a = dict(ctx=FAKE, batch=2, maxc=100, hq=32, qdt=1, q1=FAKE, q2=FAKE, qs=0, a=FAKE, ast=0,
             scale=0.0, o1=FAKE, o2=FAKE, lse=None, splits=0, ws=None, wsb=0)
    a.update(over)
    lib = _abi.lib()
    st = lib.dfx_decode_attn(ctypes.byref(k), a["ctx"], a["batch"], a["maxc"], a["hq"], a["qdt"], a["q1"],
                             a["q2"], a["qs"], a["a"], a["ast"], a["scale"], a["o1"], a["o2"], a["lse"],
                             a["splits"], a["ws"], a["wsb"], None)
    return st, lib.dfx_last_error().decode()


@pytest.mark.parametrize("kvover,over,status,needle", [
    (dict(D=96), {}, 2, "head_dim"),
    (dict(dtype=7), {}, 1, "dtype"),
    (dict(bs=24), {}, 1, "power of two"),
    (dict(heads=0), {}, 1, "num_kv_heads"),
    ({}, dict(hq=30), 1, "multiple"),
    ({}, dict(maxc=64 * 16 + 1), 1, "capacity"),
    ({}, dict(o2=None), 1, "both"),
    ({}, dict(q2=None, o2=None), 1, "without q2"),
    ({}, dict(ast=5), 1, "a_head_stride"),
    ({}, dict(qs=4100), 1, "q_batch_stride"),
    ({}, dict(q1=FAKE + 4), 1, "aligned"),
    ({}, dict(ctx=None), 1, "context_lens"),
    ({}, dict(qdt=5), 1, "q_dtype"),
    ({}, dict(splits=-1), 1, "num_splits"),
    ({}, dict(maxc=4096 + 0, splits=4), 1, "capacity"),
    (dict(mb=1024), dict(maxc=4096, splits=4, ws=None, wsb=0), 3, "workspace"),
    (dict(heads=1), dict(hq=64), 2, "query rows"),
])
def test_attention_rejects(kvover, over, status, needle):
    st, msg = attn(kv(**kvover), **over)
    assert st == status and needle in msg, (st, msg)


def test_noalloc_attention_refuses_plans_beyond_its_scratch():
    """dfx_decode_attn_noalloc checks the plan's partials against its fixed scratch array (16 MiB)
    before any HIP call, and validates its arguments as dfx_decode_attn does."""
    lib = _abi.lib()
    k = kv(mb=8192, nb=65536)
    # 64 sequences x 64 heads x 2 flows x 16 splits x 129 floats = 33.8 MB of partials
    st = lib.dfx_decode_attn_noalloc(ctypes.byref(k), FAKE, 64, 131072, 64, 1, FAKE, FAKE, 0, FAKE, 0, 0.0,
                                     FAKE, FAKE, None, 16, None)
    msg = lib.dfx_last_error().decode()
    assert st == 3 and "scratch" in msg and str(16 << 20) in msg, (st, msg)
    st = lib.dfx_decode_attn_noalloc(ctypes.byref(kv(D=96)), FAKE, 2, 100, 32, 1, FAKE, FAKE, 0, FAKE, 0, 0.0,
                                     FAKE, FAKE, None, 0, None)
    assert st == 2 and "head_dim" in lib.dfx_last_error().decode()
    st = lib.dfx_decode_attn_noalloc(ctypes.byref(k), None, 2, 100, 32, 1, FAKE, FAKE, 0, FAKE, 0, 0.0,
                                     FAKE, FAKE, None, 0, None)
    assert st == 1 and "context_lens" in lib.dfx_last_error().decode()


def test_grid_extent_limits():
    """Batches and split counts beyond a launch grid's y / z extent (65535) are refused on
    the host, before any launch."""
    lib = _abi.lib()
    st, msg = attn(kv(nb=1 << 17, mb=8), batch=65536)
    assert st == 2 and "batch" in msg
    # 65536 requested splits of a contiguous 2^22-token cache (the vector-ALU kernel's
    # 32-token quantum allows them): refused
    kc = kv(dtype=0, table=None, bs=1 << 22, nb=1, heads=1, D=64)
    st, msg = attn(kc, batch=1, maxc=1 << 22, hq=1, q2=None, o2=None, a=None, splits=65536, qdt=0)
    assert st == 2 and "splits" in msg, msg


def test_attention_workspace_size():
    """dfx_decode_attn_workspace_size: the plan's partials (every split's fp32 outputs and
    log-sum-exp values), and the plan's error paths."""
    lib = _abi.lib()
    s, n, w = ctypes.c_int32(), ctypes.c_size_t(), ctypes.c_size_t()
    k = kv(mb=8192, nb=65536)
    for batch, hq, flows, maxc, req in ((8, 64, 2, 131072, 0), (8, 64, 1, 131072, 3), (32, 32, 2, 16384, 0),
                                        (2, 32, 2, 100, 1), (0, 32, 2, 0, 0)):
        assert lib.dfx_decode_attn_workspace_size(batch, hq, flows, ctypes.byref(k), maxc, req, ctypes.byref(w)) == 0
        assert lib.dfx_decode_attn_plan(ctypes.byref(k), batch, hq, flows, maxc, req, ctypes.byref(s),
                                        ctypes.byref(n)) == 0
        assert w.value == n.value
        rows = s.value * flows * batch * hq
        if s.value == 1:
            assert w.value == 0
        else:
            up = lambda x: -(-x // 256) * 256
            assert w.value == up(rows * 128 * 4) + up(rows * 4)
    for args, needle in (((8, 64, 2, ctypes.byref(k), 131072, 0, None), "bytes"),
                         ((8, 64, 3, ctypes.byref(k), 131072, 0, ctypes.byref(w)), ""),
                         ((8, 64, 2, ctypes.byref(k), 8192 * 16 + 1, 0, ctypes.byref(w)), "capacity"),
                         ((8, 64, 2, ctypes.byref(k), 1024, -2, ctypes.byref(w)), ""),
                         ((-1, 64, 2, ctypes.byref(k), 1024, 0, ctypes.byref(w)), ""),
                         ((8, 64, 2, None, 1024, 0, ctypes.byref(w)), "kv")):
        assert lib.dfx_decode_attn_workspace_size(*args) == 1
        assert needle in lib.dfx_last_error().decode()
    bad = kv(D=96, mb=64)
    assert lib.dfx_decode_attn_workspace_size(2, 32, 2, ctypes.byref(bad), 100, 0, ctypes.byref(w)) == 2


def test_plan_is_host_arithmetic():
    lib = _abi.lib()
    s, n = ctypes.c_int32(), ctypes.c_size_t()
    k = kv(mb=8192, nb=65536)
    assert lib.dfx_decode_attn_plan(ctypes.byref(k), 8, 64, 2, 131072, 0, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value > 1 and n.value >= s.value * 2 * 8 * 64 * 129 * 4
    # a paged split holds at most 1024 blocks (its block ids sit in LDS): one requested
    # split over 131072 tokens of 16-token blocks becomes 131072 / 16384 = 8
    assert lib.dfx_decode_attn_plan(ctypes.byref(k), 8, 64, 2, 131072, 1, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 8 and n.value > 0
    # the default for this small batch: 64 (sequence, KV head) pairs, splits of 16384 tokens
    assert lib.dfx_decode_attn_plan(ctypes.byref(k), 8, 64, 2, 131072, 0, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 8
    # one (sequence, KV head) pair per CU (256 pairs): splits of at most 8192 tokens
    assert lib.dfx_decode_attn_plan(ctypes.byref(k), 32, 32, 2, 16384, 0, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 2
    # two or more pairs per CU (512): splits of at most 3072 tokens, 16384 / 2816 -> 6
    assert lib.dfx_decode_attn_plan(ctypes.byref(k), 64, 32, 2, 16384, 0, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 6
    # blocks longer than the 128-token split quantum: a split may start inside a block, so
    # it spans at most 1023 whole blocks plus the partial first one
    kb = kv(bs=256, mb=1024, nb=4096)
    assert lib.dfx_decode_attn_plan(ctypes.byref(kb), 1, 8, 1, 262144, 1, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == -(-262144 // (1023 * 256 // 128 * 128))
    kc = kv(table=None, bs=131072, nb=8)
    assert lib.dfx_decode_attn_plan(ctypes.byref(kc), 8, 64, 2, 131072, 1, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 1 and n.value == 0
    assert lib.dfx_decode_attn_plan(ctypes.byref(k), 8, 64, 2, 131072, 7, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 8          # raised to respect the 1024-block split limit
    assert lib.dfx_decode_attn_plan(ctypes.byref(k), 8, 64, 2, 131072, 20, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 20
    # fp32 caches run on the vector-ALU kernel, which walks a split one 32-token tile at a
    # time, loading the next while it multiplies the current: batch 1 x 512 tokens, 8 KV heads
    # -> splits of two tiles
    kf = kv(dtype=0, D=64, table=None, bs=512, nb=1)
    assert lib.dfx_decode_attn_plan(ctypes.byref(kf), 1, 8, 2, 512, 0, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 8 and n.value >= 8 * 2 * 8 * 65 * 4
    assert lib.dfx_decode_attn_plan(ctypes.byref(kf), 1, 8, 2, 512, 3, ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 3          # chunks of 192 tokens (a multiple of the 32-token tile)
    # so do bf16 caches with more than 16 query rows per KV head (2 flows x 16 heads)
    assert lib.dfx_decode_attn_plan(ctypes.byref(kb := kv(heads=4, nb=4096, mb=256)), 2, 64, 2, 4096, 0,
                                    ctypes.byref(s), ctypes.byref(n)) == 0
    assert s.value == 32         # 8 pairs -> 32 splits of 128 tokens
    # the plan does not depend on the number of flows while both counts use the same kernel
    # (primary results stay bit-identical)
    s1 = ctypes.c_int32()
    lib.dfx_decode_attn_plan(ctypes.byref(k), 8, 64, 1, 131072, 0, ctypes.byref(s1), ctypes.byref(n))
    lib.dfx_decode_attn_plan(ctypes.byref(k), 8, 64, 2, 131072, 0, ctypes.byref(s), ctypes.byref(n))
    assert s.value == s1.value


def test_linear_and_glue_reject():
    lib = _abi.lib()
    n = ctypes.c_size_t()
    assert lib.dfx_grouped_linear_workspace_size(3, 4, 64, 64, ctypes.byref(n)) == 1
    assert lib.dfx_grouped_linear_workspace_size(2, 4, 48, 64, ctypes.byref(n)) == 2
    assert lib.dfx_grouped_linear_workspace_size(2, 4, 64, 24, ctypes.byref(n)) == 2
    assert lib.dfx_grouped_linear_workspace_size(2, 32, 4096, 4096, ctypes.byref(n)) == 0 and n.value > 0
    st = lib.dfx_grouped_linear(2, 32, 4096, 4096, 1, FAKE, FAKE, 1, 0, FAKE, None, None, None, 0, None)
    assert st == 3 and "workspace" in lib.dfx_last_error().decode()
    assert lib.dfx_grouped_linear(2, 4, 64, 64, 9, FAKE, FAKE, 0, 0, FAKE, None, None, None, 0, None) == 1
    assert lib.dfx_grouped_linear(2, 4, 64, 64, 1, FAKE + 8, FAKE, 0, 0, FAKE, None, None, None, 0, None) == 1
    assert lib.dfx_grouped_linear(2, 4, 64, 64, 1, FAKE, FAKE, 2, 0, FAKE, None, None, None, 0, None) == 1
    assert lib.dfx_pack_weight(24, 64, FAKE, FAKE + 4096, None) == 1
    assert lib.dfx_pack_weight(32, 64, FAKE, FAKE + 1024, None) == 1      # overlapping buffers
    assert lib.dfx_rmsnorm(4, 30, FAKE, FAKE, 1e-5, FAKE, None) == 1
    assert lib.dfx_rmsnorm(4, 64, None, FAKE, 1e-5, FAKE, None) == 1
    assert lib.dfx_swiglu_couple(4, 3, 64, FAKE, None, FAKE, None) == 1       # n_flows 3
    assert lib.dfx_swiglu_couple(-1, 2, 64, FAKE, None, FAKE, None) == 1      # rows per flow < 0
    assert lib.dfx_swiglu_couple(4, 2, 62, FAKE, None, FAKE, None) == 1       # dim % 4
    assert lib.dfx_copy_bytes(FAKE, FAKE, 17, None) == 1
    assert lib.dfx_fill_bytes(FAKE + 4, 32, 0, None) == 1
    assert lib.dfx_read_bytes(FAKE, 32, None, None) == 1
    k = kv()
    assert lib.dfx_kv_append_primary(ctypes.byref(k), 2, FAKE, 0, FAKE, FAKE, 12, None) == 1
    assert lib.dfx_kv_append_primary(ctypes.byref(k), 2, FAKE, 3, FAKE, FAKE, 0, None) == 1


def test_layer_rejects():
    lib = _abi.lib()
    w = _abi.LayerWeightsStruct()
    w.hidden, w.num_q_heads, w.num_kv_heads, w.head_dim, w.intermediate, w.rms_eps = 4096, 32, 8, 128, 14336, 1e-5
    for f in ("attn_norm_gain", "w_qkv", "w_o", "mlp_norm_gain", "w_gate_up", "w_down"):
        setattr(w, f, FAKE)
    k = kv(mb=512, nb=16384)
    n = ctypes.c_size_t()
    assert lib.dfx_dual_flow_decode_layer_workspace_size(ctypes.byref(w), ctypes.byref(k), 32, 2, 8192, ctypes.byref(n)) == 0
    assert n.value > 32 * 2 * 6144 * 4
    assert lib.dfx_dual_flow_decode_layer(ctypes.byref(w), ctypes.byref(k), FAKE, 32, 8192, 2, FAKE, None, 0, None) == 3
    w.head_dim = 64
    assert lib.dfx_dual_flow_decode_layer_workspace_size(ctypes.byref(w), ctypes.byref(k), 32, 2, 8192, ctypes.byref(n)) == 1
    w.head_dim = 128
    k32 = kv(dtype=0, mb=512, nb=16384)
    assert lib.dfx_dual_flow_decode_layer_workspace_size(ctypes.byref(w), ctypes.byref(k32), 32, 2, 8192, ctypes.byref(n)) == 2


def test_layer_taps_are_disjoint_regions_of_the_workspace():
    lib = _abi.lib()
    w = _abi.LayerWeightsStruct()
    H, Hq, Hkv, D, I = 4096, 32, 8, 128, 14336
    w.hidden, w.num_q_heads, w.num_kv_heads, w.head_dim, w.intermediate, w.rms_eps = H, Hq, Hkv, D, I, 1e-5
    for f in ("attn_norm_gain", "w_qkv", "w_o", "mlp_norm_gain", "w_gate_up", "w_down"):
        setattr(w, f, FAKE)
    k = kv(mb=512, nb=16384)
    for F, B in ((2, 32), (1, 32), (2, 40), (1, 1)):
        n, t = ctypes.c_size_t(), _abi.LayerTapsStruct()
        assert lib.dfx_dual_flow_decode_layer_workspace_size(ctypes.byref(w), ctypes.byref(k), B, F, 8192, ctypes.byref(n)) == 0
        assert lib.dfx_dual_flow_decode_layer_taps(ctypes.byref(w), ctypes.byref(k), B, F, 8192, ctypes.byref(t)) == 0
        rows = -(-B // (64 // F)) * 64                     # fragment order pads to 64-row groups
        need = [("h1", rows * H * 2), ("q", F * B * (Hq + 2 * Hkv) * D * 4), ("o", rows * Hq * D * 2),
                ("h2", rows * H * 2), ("inter", rows * I * 2)]
        offs = [getattr(t, name) for name, _ in need]
        assert all(o % 256 == 0 for o in offs)
        for (name, size), start, nxt in zip(need, offs, offs[1:] + [n.value]):
            assert start + size <= nxt, (F, B, name)
    assert lib.dfx_dual_flow_decode_layer_taps(ctypes.byref(w), ctypes.byref(k), 32, 3, 8192, ctypes.byref(t)) == 1
    assert lib.dfx_dual_flow_decode_layer_taps(ctypes.byref(w), ctypes.byref(k), 32, 2, 8192, None) == 1


def test_step_rejects():
    lib = _abi.lib()
    W = _abi.LayerWeightsStruct * 2
    K = _abi.KVCacheStruct * 2
    ws, ks = W(), K()
    for w in ws:
        w.hidden, w.num_q_heads, w.num_kv_heads, w.head_dim, w.intermediate, w.rms_eps = 256, 8, 2, 64, 512, 1e-5
        for f in ("attn_norm_gain", "w_qkv", "w_o", "mlp_norm_gain", "w_gate_up", "w_down"):
            setattr(w, f, FAKE)
    ks[0], ks[1] = kv(heads=2, D=64, mb=16, nb=64), kv(heads=2, D=64, mb=16, nb=64)
    n = ctypes.c_size_t()
    assert lib.dfx_dual_flow_decode_step_workspace_size(ws, ks, 2, 4, 2, 200, ctypes.byref(n)) == 0
    n1 = ctypes.c_size_t()
    assert lib.dfx_dual_flow_decode_layer_workspace_size(ctypes.byref(ws[0]), ctypes.byref(ks[0]), 4, 2, 200, ctypes.byref(n1)) == 0
    assert n.value == n1.value                       # equal layers share one layout
    args = lambda **o: dict(dict(nl=2, tok=FAKE, vocab=10, e1=FAKE, e2=FAKE, ctx=FAKE, x=FAKE, w=FAKE, wb=n.value), **o)
    def call(**o):
        a = args(**o)
        return lib.dfx_dual_flow_decode_step(ws, ks, a["nl"], a["tok"], a["vocab"], a["e1"], a["e2"], a["ctx"], 4, 200,
                                             2, a["x"], a["w"], a["wb"], None)
    assert call(nl=0) == 1
    assert call(vocab=0) == 1
    assert call(e2=None) == 1                       # the auxiliary flow needs its own table
    assert call(e1=FAKE + 4) == 1                   # tables 8-byte aligned
    assert call(tok=None) == 1
    assert call(wb=n.value - 1) == 3
    ws[1].hidden = 512
    assert lib.dfx_dual_flow_decode_step_workspace_size(ws, ks, 2, 4, 2, 200, ctypes.byref(n)) == 1


def test_output_head_plan_and_rejects():
    lib = _abi.lib()
    n, h, lg = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    for F, B, H, V in ((2, 32, 4096, 128256), (1, 1, 64, 16), (2, 40, 256, 1040)):
        assert lib.dfx_dual_flow_output_head_workspace_size(F, B, H, V, ctypes.byref(n)) == 0
        assert lib.dfx_dual_flow_output_head_taps(F, B, H, V, ctypes.byref(h), ctypes.byref(lg)) == 0
        rows = -(-B // (64 // F)) * 64
        assert h.value == 0 and lg.value >= rows * H * 2 and lg.value % 256 == 0
        assert lg.value + F * B * V * 4 <= n.value
    assert lib.dfx_dual_flow_output_head_workspace_size(3, 4, 64, 64, ctypes.byref(n)) == 1
    assert lib.dfx_dual_flow_output_head_workspace_size(2, 4, 48, 64, ctypes.byref(n)) == 2    # hidden % 32
    assert lib.dfx_dual_flow_output_head_workspace_size(2, 4, 64, 24, ctypes.byref(n)) == 2    # vocab % 16
    assert lib.dfx_dual_flow_output_head_workspace_size(2, 70000, 64, 64, ctypes.byref(n)) == 1
    assert lib.dfx_dual_flow_output_head_workspace_size(2, 4, 64, 64, None) == 1
    assert lib.dfx_dual_flow_output_head_workspace_size(2, 4, 64, 64, ctypes.byref(n)) == 0
    need = n.value
    call = lambda x=FAKE, tok=FAKE, noise=None, ws=FAKE, wb=need, eps=1e-5: lib.dfx_dual_flow_output_head(
        2, 4, 64, 64, x, FAKE, eps, FAKE, noise, tok, None, None, ws, wb, None)
    assert call(ws=None) == 3 and "workspace" in lib.dfx_last_error().decode()
    assert call(wb=need - 1) == 3
    assert call(x=None) == 1 and call(tok=None) == 1
    assert call(x=FAKE + 4) == 1 and call(noise=FAKE + 8) == 1 and call(tok=FAKE + 2) == 1
    assert call(eps=-1.0) == 1


def moe_weights(H=4096, E=8, I=14336, k1=2, k2=2):
    w = _abi.MoeWeightsStruct()
    w.hidden, w.num_experts, w.intermediate, w.top_k_primary, w.top_k_aux, w.rms_eps = H, E, I, k1, k2, 1e-5
    for f in ("norm_gain", "w_router", "w_gate_up", "w_down"):
        setattr(w, f, FAKE)
    return w


def test_moe_plan_and_rejects():
    lib = _abi.lib()
    n, t = ctypes.c_size_t(), _abi.MoeTapsStruct()
    for F, B, E, I in ((2, 32, 8, 14336), (1, 32, 8, 14336), (2, 40, 2, 128), (2, 3, 16, 2048)):
        w = moe_weights(H=256 if I < 4096 else 4096, E=E, I=I)
        H = w.hidden
        assert lib.dfx_dual_flow_moe_mlp_workspace_size(ctypes.byref(w), B, F, ctypes.byref(n)) == 0
        assert lib.dfx_dual_flow_moe_mlp_taps(ctypes.byref(w), B, F, ctypes.byref(t)) == 0
        groups = -(-B // (64 // F))
        assert t.inter_stride == groups * 64 * I
        offs = [t.h, t.logits, t.ids, t.weights, t.counts, t.seqs, t.inter]
        sizes = [F * B * H * 2, F * B * E * 4, F * B * 64, F * B * 64, E * 4, E * B * 4, E * t.inter_stride * 2]
        assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
        for o, s, nxt in zip(offs, sizes, offs[1:] + [n.value]):
            assert o + s <= nxt
    bad = [dict(E=0), dict(E=257), dict(k1=0), dict(k1=17, E=32), dict(k1=9, E=8), dict(k2=0), dict(I=48), dict(H=48)]
    for kw in bad:
        w = moe_weights(**kw)
        assert lib.dfx_dual_flow_moe_mlp_workspace_size(ctypes.byref(w), 4, 2, ctypes.byref(n)) != 0, kw
    w = moe_weights(k2=0)
    assert lib.dfx_dual_flow_moe_mlp_workspace_size(ctypes.byref(w), 4, 1, ctypes.byref(n)) == 0   # k2 unused
    w = moe_weights(E=256)
    assert lib.dfx_dual_flow_moe_mlp_workspace_size(ctypes.byref(w), 2048, 2, ctypes.byref(n)) == 0
    assert lib.dfx_dual_flow_moe_mlp_workspace_size(ctypes.byref(w), 2049, 2, ctypes.byref(n)) == 2  # LDS bitmap
    w = moe_weights()
    w.w_router = FAKE + 8
    assert lib.dfx_dual_flow_moe_mlp_workspace_size(ctypes.byref(w), 4, 2, ctypes.byref(n)) == 1
    w = moe_weights()
    assert lib.dfx_dual_flow_moe_mlp_workspace_size(ctypes.byref(w), 4, 2, ctypes.byref(n)) == 0
    assert lib.dfx_dual_flow_moe_mlp(ctypes.byref(w), 4, 2, FAKE, None, 0, None) == 3
    assert lib.dfx_dual_flow_moe_mlp(ctypes.byref(w), 4, 2, FAKE + 4, FAKE, n.value, None) == 1
    assert lib.dfx_dual_flow_moe_mlp(ctypes.byref(w), 4, 2, None, FAKE, n.value, None) == 1
    assert lib.dfx_dual_flow_moe_mlp(None, 4, 2, FAKE, FAKE, n.value, None) == 1


def test_prefill_rejects():
    lib = _abi.lib()
    w = _abi.LayerWeightsStruct()
    w.hidden, w.num_q_heads, w.num_kv_heads, w.head_dim, w.intermediate, w.rms_eps = 4096, 32, 8, 128, 14336, 1e-5
    for f in ("attn_norm_gain", "w_qkv", "w_o", "mlp_norm_gain", "w_gate_up", "w_down"):
        setattr(w, f, FAKE)
    k = kv(mb=512, nb=16384)
    n = ctypes.c_size_t()
    assert lib.dfx_prefill_layer_workspace_size(ctypes.byref(w), ctypes.byref(k), 2, 2048, 8192, ctypes.byref(n)) == 0
    rows = 2 * 2048
    assert n.value >= rows * (32 + 16) * 128 * 4 + 3 * rows * 4096 * 2 + rows * 14336 * 2
    assert lib.dfx_prefill_layer_workspace_size(ctypes.byref(w), ctypes.byref(k), 2, 2048, 8193 * 8, ctypes.byref(n)) == 1
    assert lib.dfx_prefill_layer(ctypes.byref(w), ctypes.byref(k), FAKE, 2, 2048, 8192, FAKE, None, 0, None) == 3
    assert lib.dfx_prefill_layer(ctypes.byref(w), ctypes.byref(k), FAKE, 2, 0, 8192, FAKE, None, 0, None) == 0
    # the intermediates' offsets: regions in order h1, q, o, h2, inter, inside the workspace
    t = _abi.LayerTapsStruct()
    assert lib.dfx_prefill_layer_taps(ctypes.byref(w), ctypes.byref(k), 2, 2048, 8192, ctypes.byref(t)) == 0
    assert t.h1 == 0 and t.q >= rows * 4096 * 2 and t.o >= t.q + rows * (32 + 16) * 128 * 4
    assert t.h2 >= t.o + rows * 32 * 128 * 2 and t.inter >= t.h2 + rows * 4096 * 2
    assert t.inter + rows * 14336 * 2 <= n.value
    assert lib.dfx_prefill_layer_taps(ctypes.byref(w), ctypes.byref(k), 2, 2048, 8192, None) == 1
    assert lib.dfx_prefill_layer_taps(ctypes.byref(w), ctypes.byref(k), 2, 2048, 8193 * 8, ctypes.byref(t)) == 1
    w.num_q_heads = 6
    assert lib.dfx_prefill_layer_workspace_size(ctypes.byref(w), ctypes.byref(k), 2, 16, 8192, ctypes.byref(n)) == 2
    k32 = kv(dtype=0, mb=512, nb=16384)
    assert lib.dfx_prefill_attn(ctypes.byref(k32), FAKE, 2, 16, 64, 32, FAKE, 0, FAKE, None, None) == 2
    assert lib.dfx_prefill_attn(ctypes.byref(k), FAKE, 2, 16, 64, 32, FAKE, 100, FAKE, None, None) == 1  # stride
    assert lib.dfx_prefill_attn(ctypes.byref(k), FAKE, 2, 16, 64, 32, FAKE + 4, 0, FAKE, None, None) == 1
    assert lib.dfx_prefill_attn(ctypes.byref(k), FAKE, 2, 16, 64, 30, FAKE, 0, FAKE, None, None) == 2    # heads
    assert lib.dfx_prefill_attn(ctypes.byref(k), FAKE, 1 << 16, 16, 64, 32, FAKE, 0, FAKE, None, None) == 1
    kbig = kv(mb=1 << 17, nb=1 << 17)
    assert lib.dfx_prefill_attn(ctypes.byref(kbig), FAKE, 1, 65535 * 16 + 1, 1 << 21, 32, FAKE, 0, FAKE, None, None) == 2
    # both flows: the same limits, plus the auxiliary's query, output and coupling stride
    dual = lambda kk, **o: lib.dfx_prefill_dual_attn(
        ctypes.byref(kk), FAKE, o.get("B", 2), 16, 64, o.get("hq", 32), FAKE, o.get("q2", FAKE), o.get("a", FAKE),
        o.get("ast", 0), 0, FAKE, o.get("o2", FAKE), None, None)
    assert dual(k32) == 2
    assert dual(k, hq=30) == 2
    assert dual(k, q2=None) == 1 and "q2_raw" in lib.dfx_last_error().decode()
    assert dual(k, o2=None) == 1
    assert dual(k, ast=64) == 1 and "a_head_stride" in lib.dfx_last_error().decode()
    assert dual(k, a=FAKE + 2) == 1
    assert dual(k, B=0, q2=None) == 0          # nothing to do: no pointer is read
    W = _abi.LayerWeightsStruct * 1
    K = _abi.KVCacheStruct * 1
    ws, ks = W(), K()
    ws[0], ks[0] = w, k
    ws[0].num_q_heads = 32
    assert lib.dfx_prefill_step_workspace_size(ws, ks, 1, 2, 16, 64, ctypes.byref(n)) == 0
    assert lib.dfx_prefill_step(ws, ks, 1, FAKE, 0, FAKE, FAKE, 2, 16, 64, FAKE, FAKE, n.value, None) == 1
    assert lib.dfx_prefill_step(ws, ks, 0, FAKE, 10, FAKE, FAKE, 2, 16, 64, FAKE, FAKE, n.value, None) == 1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with status 2 and says so, before
    touching a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(HEADER), "..", "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
