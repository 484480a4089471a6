"""dual_flow_shared_amd -- the dual-flow decode step on MI355X (gfx950).

Thin torch-facing binding of libdfx.so (include/dfx.h): it checks shapes and dtypes,
passes device pointers and the current HIP stream, and returns torch tensors. Every
step of the path runs in the library's HIP kernels; torch only holds device memory.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from ._abi import (DFX_BF16, DFX_F32, DFX_W_PACKED, DFX_W_ROW_MAJOR, DfxError, KVCacheStruct,
                   LayerTapsStruct, LayerWeightsStruct, MoeTapsStruct, MoeWeightsStruct, check, lib)

__all__ = ["DfxError", "KVCache", "LayerWeights", "decode_attn", "decode_attn_plan", "decode_attn_workspace_size",
           "kv_append_primary", "grouped_linear", "pack_weight", "rmsnorm", "swiglu_couple",
           "dual_flow_decode_layer", "layer_workspace_size", "copy_bytes", "read_bytes", "fill_bytes",
           "layer_taps", "dual_flow_decode_step", "step_workspace_size", "output_head",
           "output_head_workspace_size", "output_head_taps", "MoeWeights", "moe_mlp", "moe_workspace_size",
           "moe_taps", "prefill_attn", "prefill_layer", "prefill_layer_taps", "prefill_step", "Workspace", "version"]


def version() -> int:
    return lib().dfx_version()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DFX_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return DFX_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _contig(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class Workspace:
    """A device byte buffer grown on demand (scratch for the library's split partials and
    the layer's intermediates)."""

    def __init__(self, device=None):
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self.buf = torch.zeros(0, dtype=torch.uint8, device=self.device)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 2 * self.buf.numel()), dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def _workspace(ws: Optional[Workspace], device, purpose: str) -> Workspace:
    """Default workspaces are kept per device and per purpose, so that the intermediates a
    layer call leaves in its workspace survive later calls of other entry points."""
    if ws is not None:
        return ws
    d = torch.device(device)
    key = (d.index if d.index is not None else torch.cuda.current_device(), purpose)
    if key not in _default_ws:
        _default_ws[key] = Workspace(torch.device("cuda", key[0]))
    return _default_ws[key]


@dataclass
class KVCache:
    """The primary flow's persistent K/V pool [num_blocks][Hkv][block_size][D]
    (bfloat16 or float32) with an optional int32 block table [batch][max_blocks]."""
    k: torch.Tensor
    v: torch.Tensor
    block_table: Optional[torch.Tensor] = None

    def struct(self) -> KVCacheStruct:
        k, v = _contig(self.k, "k"), _contig(self.v, "v")
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
            raise ValueError("k and v must be equal-shaped [blocks][Hkv][block_size][D] tensors")
        s = KVCacheStruct()
        s.dtype = _dtype_code(k)
        s.num_blocks, s.num_kv_heads, s.block_size, s.head_dim = k.shape
        s.k, s.v = k.data_ptr(), v.data_ptr()
        if self.block_table is not None:
            bt = _contig(self.block_table, "block_table")
            if bt.dtype != torch.int32 or bt.dim() != 2:
                raise ValueError("block_table must be int32 [batch][max_blocks]")
            s.block_table, s.max_blocks_per_seq = bt.data_ptr(), bt.shape[1]
        else:
            s.block_table, s.max_blocks_per_seq = None, 0
        s.reserved = 0
        return s

    @property
    def capacity(self) -> int:
        bs = self.k.shape[2]
        return bs * self.block_table.shape[1] if self.block_table is not None else bs


def decode_attn_plan(cache: KVCache, batch: int, num_q_heads: int, n_flows: int, max_context: int,
                     num_splits: int = 0):
    s = ctypes.c_int32()
    n = ctypes.c_size_t()
    st = cache.struct()
    check(lib().dfx_decode_attn_plan(ctypes.byref(st), batch, num_q_heads, n_flows, max_context,
                                     num_splits, ctypes.byref(s), ctypes.byref(n)))
    return s.value, n.value


def decode_attn_workspace_size(cache: KVCache, batch: int, num_q_heads: int, n_flows: int, max_context: int,
                               num_splits: int = 0) -> int:
    n = ctypes.c_size_t()
    st = cache.struct()
    check(lib().dfx_decode_attn_workspace_size(batch, num_q_heads, n_flows, ctypes.byref(st), max_context,
                                               num_splits, ctypes.byref(n)))
    return n.value


def decode_attn(q1: torch.Tensor, q2_raw: Optional[torch.Tensor] = None, a: Optional[torch.Tensor] = None,
                *, cache: KVCache, context_lens: torch.Tensor, max_context: int, num_splits: int = 0,
                softmax_scale: float = 0.0, want_lse: bool = True, out=None,
                workspace: Optional[Workspace] = None, stream=None):
    """Dual-query decode attention (dfx_decode_attn). q1, q2_raw: [B][Hq][D] (rows may be
    strided: the batch stride is taken from the tensor). a: fp32 [D] or [Hq][D].
    Returns (o1, o2 or None, lse [F][B][Hq] or None)."""
    B, Hq, D = q1.shape
    if q1.stride(2) != 1 or q1.stride(1) != D:
        raise ValueError("q1 rows must be [Hq][D] contiguous within a sequence")
    if q2_raw is not None and (q2_raw.shape != q1.shape or q2_raw.stride() != q1.stride()
                               or q2_raw.dtype != q1.dtype):
        raise ValueError("q2_raw must match q1 in shape, strides and dtype")
    F = 1 if q2_raw is None else 2
    if context_lens.dtype != torch.int32 or context_lens.numel() != B:
        raise ValueError("context_lens must be int32 [batch]")
    a_stride = 0
    if a is not None:
        if a.dtype != torch.float32:
            raise TypeError("a must be float32")
        a = _contig(a, "a")
        a_stride = 0 if a.numel() == D else D
        if a.numel() not in (D, Hq * D):
            raise ValueError("a must be [D] or [Hq][D]")
    dev = q1.device
    if out is None:
        o1 = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
        o2 = torch.empty(B, Hq, D, dtype=torch.float32, device=dev) if F == 2 else None
    else:
        o1, o2 = out
    lse = torch.empty(F, B, Hq, dtype=torch.float32, device=dev) if want_lse else None
    if cache.block_table is not None and cache.block_table.shape[0] < B:
        raise ValueError("block_table has fewer rows than the batch")
    st = cache.struct()
    splits, need = decode_attn_plan(cache, B, Hq, F, max_context, num_splits)
    ws = _workspace(workspace, dev, "attn").get(need) if need else None
    check(lib().dfx_decode_attn(ctypes.byref(st), _ptr(context_lens), B, max_context, Hq, _dtype_code(q1),
                                _ptr(q1), _ptr(q2_raw), q1.stride(0), _ptr(a), a_stride,
                                float(softmax_scale), _ptr(o1), _ptr(o2), _ptr(lse), num_splits,
                                _ptr(ws), need, _stream(stream)))
    return o1, o2, lse


def kv_append_primary(cache: KVCache, positions: torch.Tensor, k_new: torch.Tensor,
                      v_new: torch.Tensor, stream=None) -> None:
    """Write the primary rows k_new, v_new ([B][Hkv*D], row stride from the tensor) at
    positions[b] (dfx_kv_append_primary)."""
    B = positions.numel()
    if positions.dtype != torch.int32:
        raise ValueError("positions must be int32")
    if k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype or k_new.stride(-1) != 1:
        raise ValueError("k_new and v_new must share dtype and row-major strides")
    st = cache.struct()
    check(lib().dfx_kv_append_primary(ctypes.byref(st), B, _ptr(positions), _dtype_code(k_new),
                                      _ptr(k_new), _ptr(v_new), k_new.stride(0), _stream(stream)))


def pack_weight(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Row-major bf16 W [N][K] -> the same matrix in DFX_W_PACKED fragment order (a new
    [N][K]-sized tensor; the shape is kept for bookkeeping, the element order is not)."""
    w = _contig(w, "w")
    N, K = w.shape
    out = torch.empty_like(w)
    check(lib().dfx_pack_weight(N, K, _ptr(w), _ptr(out), _stream(stream)))
    return out


def grouped_linear(x: torch.Tensor, w: torch.Tensor, *, packed: bool = False, y_dtype=torch.float32,
                   couple: Optional[torch.Tensor] = None, residual: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None,
                   stream=None) -> torch.Tensor:
    """Y[f] = bf16(X[f]) W^T (+ couple, + residual) for x [F][rows][K], w bf16 [N][K]
    (row-major, or packed by pack_weight when ``packed``)."""
    F, rows, K = x.shape
    N = w.shape[0]
    x, w = _contig(x, "x"), _contig(w, "w")
    if w.shape[1] != K:
        raise ValueError("w must be [N][K]")
    y = out if out is not None else torch.empty(F, rows, N, dtype=y_dtype, device=x.device)
    n = ctypes.c_size_t()
    check(lib().dfx_grouped_linear_workspace_size(F, rows, K, N, ctypes.byref(n)))
    ws = _workspace(workspace, x.device, "linear").get(n.value) if n.value else None
    check(lib().dfx_grouped_linear(F, rows, K, N, _dtype_code(x), _ptr(x), _ptr(w),
                                   DFX_W_PACKED if packed else DFX_W_ROW_MAJOR, _dtype_code(y),
                                   _ptr(y), _ptr(couple), _ptr(residual), _ptr(ws), n.value,
                                   _stream(stream)))
    return y


def rmsnorm(x: torch.Tensor, gain: torch.Tensor, eps: float, out=None, stream=None) -> torch.Tensor:
    x = _contig(x, "x")
    dim = x.shape[-1]
    rows = x.numel() // dim
    y = out if out is not None else torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    check(lib().dfx_rmsnorm(rows, dim, _ptr(x), _ptr(gain), float(eps), _ptr(y), _stream(stream)))
    return y


def swiglu_couple(gate_up: torch.Tensor, b: Optional[torch.Tensor] = None, out=None,
                  stream=None) -> torch.Tensor:
    gate_up = _contig(gate_up, "gate_up")
    F, rows, two_i = gate_up.shape
    y = out if out is not None else torch.empty(F, rows, two_i // 2, dtype=torch.bfloat16,
                                                device=gate_up.device)
    check(lib().dfx_swiglu_couple(rows, F, two_i // 2, _ptr(gate_up), _ptr(b), _ptr(y), _stream(stream)))
    return y


@dataclass
class LayerWeights:
    """Device weights of one dual-flow layer: the four matrices bf16 [out][in] in packed
    fragment order (see ``LayerWeights.from_row_major``), vectors fp32."""
    attn_norm_gain: torch.Tensor
    w_qkv: torch.Tensor
    w_o: torch.Tensor
    mlp_norm_gain: torch.Tensor
    w_gate_up: torch.Tensor
    w_down: torch.Tensor
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    eps: float = 1e-5
    couple_a: Optional[torch.Tensor] = None
    couple_b: Optional[torch.Tensor] = None
    couple_c: Optional[torch.Tensor] = None

    @classmethod
    def from_row_major(cls, attn_norm_gain, w_qkv, w_o, mlp_norm_gain, w_gate_up, w_down,
                       num_q_heads, num_kv_heads, head_dim, eps=1e-5, couple_a=None, couple_b=None,
                       couple_c=None) -> "LayerWeights":
        """Pack row-major device matrices once (dfx_pack_weight) and keep the packed copies."""
        return cls(attn_norm_gain, pack_weight(w_qkv), pack_weight(w_o), mlp_norm_gain,
                   pack_weight(w_gate_up), pack_weight(w_down), num_q_heads, num_kv_heads,
                   head_dim, eps, couple_a, couple_b, couple_c)

    def struct(self) -> LayerWeightsStruct:
        s = LayerWeightsStruct()
        s.hidden = self.w_qkv.shape[1]
        s.num_q_heads, s.num_kv_heads, s.head_dim = self.num_q_heads, self.num_kv_heads, self.head_dim
        s.intermediate = self.w_down.shape[1]
        s.rms_eps = self.eps
        for name in ("attn_norm_gain", "w_qkv", "w_o", "mlp_norm_gain", "w_gate_up", "w_down",
                     "couple_a", "couple_b", "couple_c"):
            t = getattr(self, name)
            setattr(s, name, None if t is None else _contig(t, name).data_ptr())
        return s


def layer_workspace_size(weights: LayerWeights, cache: KVCache, batch: int, n_flows: int,
                         max_context: int) -> int:
    n = ctypes.c_size_t()
    w, c = weights.struct(), cache.struct()
    check(lib().dfx_dual_flow_decode_layer_workspace_size(ctypes.byref(w), ctypes.byref(c), batch,
                                                          n_flows, max_context, ctypes.byref(n)))
    return n.value


def dual_flow_decode_layer(x: torch.Tensor, weights: LayerWeights, cache: KVCache,
                           context_lens: torch.Tensor, max_context: int,
                           workspace: Optional[Workspace] = None, stream=None) -> torch.Tensor:
    """One decode step of one layer, in place on x [F][B][hidden] fp32 (F = 2: both flows)."""
    F, B, H = x.shape
    x = _contig(x, "x")
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    w, c = weights.struct(), cache.struct()
    need = layer_workspace_size(weights, cache, B, F, max_context)
    ws = _workspace(workspace, x.device, "layer").get(need)
    check(lib().dfx_dual_flow_decode_layer(ctypes.byref(w), ctypes.byref(c), _ptr(context_lens), B,
                                           max_context, F, _ptr(x), _ptr(ws), need, _stream(stream)))
    return x


def _structs(layers, caches):
    if len(layers) != len(caches) or not layers:
        raise ValueError("one cache per layer, at least one layer")
    ws = (LayerWeightsStruct * len(layers))(*[w.struct() for w in layers])
    cs = (KVCacheStruct * len(caches))(*[c.struct() for c in caches])
    return ws, cs


def step_workspace_size(layers, caches, batch: int, n_flows: int, max_context: int) -> int:
    n = ctypes.c_size_t()
    ws, cs = _structs(layers, caches)
    check(lib().dfx_dual_flow_decode_step_workspace_size(ws, cs, len(layers), batch, n_flows, max_context,
                                                          ctypes.byref(n)))
    return n.value


def dual_flow_decode_step(tokens: torch.Tensor, embed_primary: torch.Tensor, embed_aux: Optional[torch.Tensor],
                          layers, caches, context_lens: torch.Tensor, max_context: int, n_flows: int = 2,
                          out: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None,
                          stream=None) -> torch.Tensor:
    """One decode step of a layer stack: token ids [B] int32 -> residual rows [F][B][hidden]
    fp32 after the last layer (each layer appends the primary's K/V row to its own cache)."""
    tokens = _contig(tokens, "tokens")
    if tokens.dtype != torch.int32:
        raise TypeError("tokens must be int32")
    B = tokens.numel()
    vocab, H = embed_primary.shape
    x = out if out is not None else torch.empty(n_flows, B, H, dtype=torch.float32, device=tokens.device)
    ws, cs = _structs(layers, caches)
    need = step_workspace_size(layers, caches, B, n_flows, max_context)
    buf = _workspace(workspace, tokens.device, "step").get(need)
    check(lib().dfx_dual_flow_decode_step(ws, cs, len(layers), _ptr(tokens), vocab, _ptr(_contig(embed_primary, "embed_primary")),
                                          None if embed_aux is None else _ptr(_contig(embed_aux, "embed_aux")),
                                          _ptr(context_lens), B, max_context, n_flows, _ptr(x), _ptr(buf), need,
                                          _stream(stream)))
    return x


def layer_taps(weights: LayerWeights, cache: KVCache, batch: int, n_flows: int,
               max_context: int) -> dict:
    """Byte offsets of a layer call's intermediates in its workspace: h1, q, o, h2, inter
    (layouts in include/dfx.h, dfx_dual_flow_decode_layer_taps)."""
    t = LayerTapsStruct()
    w, c = weights.struct(), cache.struct()
    check(lib().dfx_dual_flow_decode_layer_taps(ctypes.byref(w), ctypes.byref(c), batch, n_flows,
                                                max_context, ctypes.byref(t)))
    return {name: getattr(t, name) for name, _ in t._fields_}


def output_head_workspace_size(n_flows: int, batch: int, hidden: int, vocab: int) -> int:
    n = ctypes.c_size_t()
    check(lib().dfx_dual_flow_output_head_workspace_size(n_flows, batch, hidden, vocab, ctypes.byref(n)))
    return n.value


def output_head_taps(n_flows: int, batch: int, hidden: int, vocab: int) -> dict:
    """Byte offsets of the head's normed rows (fragment order) and fp32 logits in its workspace."""
    h, lg = ctypes.c_size_t(), ctypes.c_size_t()
    check(lib().dfx_dual_flow_output_head_taps(n_flows, batch, hidden, vocab, ctypes.byref(h), ctypes.byref(lg)))
    return {"h": h.value, "logits": lg.value}


def output_head(x: torch.Tensor, norm_gain: torch.Tensor, eps: float, w_out_packed: torch.Tensor,
                uniform_noise: Optional[torch.Tensor] = None, *, want_p_mix: bool = False,
                workspace: Optional[Workspace] = None, stream=None):
    """Shared output head and flow mixture: x [F][B][hidden] fp32 after the last layer ->
    (next_token [B] int32, alpha [B] fp32, p_mix [B][V] fp32 or None). w_out_packed: the
    [vocab][hidden] bf16 matrix in packed layout (pack_weight). uniform_noise [B][V] fp32 in
    (0, 1) makes the token a Gumbel-max draw from p_mix; None is greedy."""
    x = _contig(x, "x")
    if x.dim() != 3 or x.dtype != torch.float32:
        raise ValueError("x must be fp32 [n_flows][batch][hidden]")
    F, B, H = x.shape
    V = w_out_packed.numel() // H
    if w_out_packed.numel() != V * H:
        raise ValueError("w_out_packed size is not a multiple of hidden")
    dev = x.device
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    alpha = torch.empty(B, dtype=torch.float32, device=dev)
    p_mix = torch.empty(B, V, dtype=torch.float32, device=dev) if want_p_mix else None
    if uniform_noise is not None:
        uniform_noise = _contig(uniform_noise, "uniform_noise")
        if uniform_noise.shape != (B, V) or uniform_noise.dtype != torch.float32:
            raise ValueError("uniform_noise must be fp32 [batch][vocab]")
    need = output_head_workspace_size(F, B, H, V)
    buf = _workspace(workspace, dev, "head").get(need)
    check(lib().dfx_dual_flow_output_head(F, B, H, V, _ptr(x), _ptr(_contig(norm_gain, "norm_gain")), eps,
                                          _ptr(_contig(w_out_packed, "w_out_packed")), _ptr(uniform_noise),
                                          _ptr(tok), _ptr(alpha), _ptr(p_mix), _ptr(buf), need, _stream(stream)))
    return tok, alpha, p_mix


@dataclass
class MoeWeights:
    """Device weights of a mixture-of-experts MLP block: router bf16 [E][hidden] row-major;
    per-expert gate/up [E][2I][hidden] and down [E][hidden][I] bf16 in packed fragment order
    (``MoeWeights.from_row_major``); vectors fp32."""
    norm_gain: torch.Tensor
    w_router: torch.Tensor
    w_gate_up: torch.Tensor
    w_down: torch.Tensor
    top_k_primary: int
    top_k_aux: int
    eps: float = 1e-5
    couple_b: Optional[torch.Tensor] = None
    couple_c: Optional[torch.Tensor] = None

    @classmethod
    def from_row_major(cls, norm_gain, w_router, w_gate_up, w_down, top_k_primary, top_k_aux, eps=1e-5,
                       couple_b=None, couple_c=None) -> "MoeWeights":
        """Pack every expert's row-major matrices once (dfx_pack_weight per expert)."""
        gu = torch.stack([pack_weight(w_gate_up[e]) for e in range(w_gate_up.shape[0])])
        dn = torch.stack([pack_weight(w_down[e]) for e in range(w_down.shape[0])])
        return cls(norm_gain, _contig(w_router, "w_router"), gu, dn, top_k_primary, top_k_aux, eps,
                   couple_b, couple_c)

    def struct(self) -> MoeWeightsStruct:
        s = MoeWeightsStruct()
        s.num_experts, s.hidden, s.intermediate = self.w_down.shape
        s.top_k_primary, s.top_k_aux, s.rms_eps = self.top_k_primary, self.top_k_aux, self.eps
        for name in ("norm_gain", "w_router", "w_gate_up", "w_down", "couple_b", "couple_c"):
            t = getattr(self, name)
            setattr(s, name, None if t is None else _contig(t, name).data_ptr())
        return s


def moe_workspace_size(weights: MoeWeights, batch: int, n_flows: int) -> int:
    n = ctypes.c_size_t()
    w = weights.struct()
    check(lib().dfx_dual_flow_moe_mlp_workspace_size(ctypes.byref(w), batch, n_flows, ctypes.byref(n)))
    return n.value


def moe_taps(weights: MoeWeights, batch: int, n_flows: int) -> dict:
    """Byte offsets of the MoE block's intermediates in its workspace (include/dfx.h)."""
    t = MoeTapsStruct()
    w = weights.struct()
    check(lib().dfx_dual_flow_moe_mlp_taps(ctypes.byref(w), batch, n_flows, ctypes.byref(t)))
    return {name: getattr(t, name) for name, _ in t._fields_}


def moe_mlp(x: torch.Tensor, weights: MoeWeights, workspace: Optional[Workspace] = None,
            stream=None) -> torch.Tensor:
    """The mixture-of-experts MLP block with router replay, in place on x [F][B][hidden] fp32."""
    x = _contig(x, "x")
    if x.dim() != 3 or x.dtype != torch.float32:
        raise ValueError("x must be fp32 [n_flows][batch][hidden]")
    F, B, H = x.shape
    w = weights.struct()
    if w.hidden != H:
        raise ValueError("x and the weights disagree on hidden")
    need = moe_workspace_size(weights, B, F)
    buf = _workspace(workspace, x.device, "moe").get(need)
    check(lib().dfx_dual_flow_moe_mlp(ctypes.byref(w), B, F, _ptr(x), _ptr(buf), need, _stream(stream)))
    return x


def prefill_attn(q: torch.Tensor, cache: KVCache, start_pos: torch.Tensor, max_context: int,
                 want_lse: bool = False, stream=None):
    """Causal attention of a prompt chunk, q fp32 [B][T][Hq][D] (keys and values of the chunk
    already in the cache at start_pos[b] + t) -> o fp32 [B][T][Hq][D] (and lse [B][T][Hq])."""
    q = _contig(q, "q")
    if q.dim() != 4 or q.dtype != torch.float32:
        raise ValueError("q must be fp32 [batch][chunk][heads][head_dim]")
    B, T, Hq, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, T, Hq, dtype=torch.float32, device=q.device) if want_lse else None
    c = cache.struct()
    check(lib().dfx_prefill_attn(ctypes.byref(c), _ptr(start_pos), B, T, max_context, Hq, _ptr(q), 0, _ptr(o),
                                 _ptr(lse), _stream(stream)))
    return (o, lse) if want_lse else o


def prefill_dual_attn(q1: torch.Tensor, q2_raw: torch.Tensor, a: Optional[torch.Tensor], cache: KVCache,
                      start_pos: torch.Tensor, max_context: int, want_lse: bool = False, stream=None):
    """Causal attention of a chunk with both flows at every position (the training-time
    forward): q1, q2_raw fp32 [B][T][Hq][D], a fp32 [D] or [Hq][D] or None (Q2 = q2_raw + a * Q1)
    -> o1, o2 fp32 [B][T][Hq][D] (and lse [2][B][T][Hq])."""
    q1, q2_raw = _contig(q1, "q1"), _contig(q2_raw, "q2_raw")
    if q1.dim() != 4 or q1.dtype != torch.float32 or q2_raw.shape != q1.shape or q2_raw.dtype != torch.float32:
        raise ValueError("q1 and q2_raw must be fp32 [batch][chunk][heads][head_dim] of one shape")
    B, T, Hq, D = q1.shape
    stride = 0
    if a is not None:
        a = _contig(a, "a")
        if a.dtype != torch.float32 or a.numel() not in (D, Hq * D):
            raise ValueError("a must be fp32 [head_dim] or [heads][head_dim]")
        stride = 0 if a.numel() == D else D
    o1, o2 = torch.empty_like(q1), torch.empty_like(q1)
    lse = torch.empty(2, B, T, Hq, dtype=torch.float32, device=q1.device) if want_lse else None
    c = cache.struct()
    check(lib().dfx_prefill_dual_attn(ctypes.byref(c), _ptr(start_pos), B, T, max_context, Hq, _ptr(q1), _ptr(q2_raw),
                                      _ptr(a), stride, 0, _ptr(o1), _ptr(o2), _ptr(lse), _stream(stream)))
    return (o1, o2, lse) if want_lse else (o1, o2)


def prefill_layer_taps(weights: LayerWeights, cache: KVCache, batch: int, chunk: int, max_context: int) -> dict:
    """Byte offsets of a prefill layer call's intermediates in its workspace: h1, q, o, h2, inter
    (layouts in include/dfx.h, dfx_prefill_layer_taps)."""
    t = LayerTapsStruct()
    w, c = weights.struct(), cache.struct()
    check(lib().dfx_prefill_layer_taps(ctypes.byref(w), ctypes.byref(c), batch, chunk, max_context, ctypes.byref(t)))
    return {name: getattr(t, name) for name, _ in t._fields_}


def prefill_layer(x: torch.Tensor, weights: LayerWeights, cache: KVCache, start_pos: torch.Tensor,
                  max_context: int, workspace: Optional[Workspace] = None, stream=None) -> torch.Tensor:
    """One layer of the primary over a prompt chunk, in place on x [B][T][hidden] fp32."""
    x = _contig(x, "x")
    if x.dim() != 3 or x.dtype != torch.float32:
        raise ValueError("x must be fp32 [batch][chunk][hidden]")
    B, T, _ = x.shape
    w, c = weights.struct(), cache.struct()
    n = ctypes.c_size_t()
    check(lib().dfx_prefill_layer_workspace_size(ctypes.byref(w), ctypes.byref(c), B, T, max_context,
                                                 ctypes.byref(n)))
    buf = _workspace(workspace, x.device, "prefill").get(n.value)
    check(lib().dfx_prefill_layer(ctypes.byref(w), ctypes.byref(c), _ptr(start_pos), B, T, max_context, _ptr(x),
                                  _ptr(buf), n.value, _stream(stream)))
    return x


def prefill_step(tokens: torch.Tensor, embed_primary: torch.Tensor, layers, caches, start_pos: torch.Tensor,
                 max_context: int, out: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None,
                 stream=None) -> torch.Tensor:
    """A prompt chunk through the primary's embeddings and every layer: tokens int32 [B][T] ->
    residual rows [B][T][hidden] fp32 (each layer appends the chunk's keys and values)."""
    tokens = _contig(tokens, "tokens")
    if tokens.dim() != 2 or tokens.dtype != torch.int32:
        raise ValueError("tokens must be int32 [batch][chunk]")
    B, T = tokens.shape
    vocab, H = embed_primary.shape
    x = out if out is not None else torch.empty(B, T, H, dtype=torch.float32, device=tokens.device)
    ws, cs = _structs(layers, caches)
    n = ctypes.c_size_t()
    check(lib().dfx_prefill_step_workspace_size(ws, cs, len(layers), B, T, max_context, ctypes.byref(n)))
    buf = _workspace(workspace, tokens.device, "prefill").get(n.value)
    check(lib().dfx_prefill_step(ws, cs, len(layers), _ptr(tokens), vocab, _ptr(_contig(embed_primary, "embed_primary")),
                                 _ptr(start_pos), B, T, max_context, _ptr(x), _ptr(buf), n.value, _stream(stream)))
    return x


def copy_bytes(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    n = min(dst.numel() * dst.element_size(), src.numel() * src.element_size())
    check(lib().dfx_copy_bytes(_ptr(dst), _ptr(src), n - n % 16, _stream(stream)))


def read_bytes(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Read every byte of src once on the GPU (achievable read bandwidth)."""
    if sink is None:
        sink = torch.empty(4096 * 256, dtype=torch.int32, device=src.device)
    n = src.numel() * src.element_size()
    check(lib().dfx_read_bytes(_ptr(src), n - n % 16, _ptr(sink), _stream(stream)))
    return sink


def fill_bytes(dst: torch.Tensor, pattern: int = 0, stream=None) -> None:
    n = dst.numel() * dst.element_size()
    check(lib().dfx_fill_bytes(_ptr(dst), n - n % 16, pattern, _stream(stream)))
