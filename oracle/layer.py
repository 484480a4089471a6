"""One dual-flow decode layer (oracle, fp64 with bf16 rounding at five fixed points).

Structure (Sintesi Tecnica: Dual-Flow Transformers, "Architettura Core" and
"Meccanismi Chiave"): two residual rows per sequence at the generated
position -- flow 0 primary, flow 1 auxiliary -- pass through the same norm
gains and matrices. Only the primary's key/value row is appended to the
cache; both flows' queries attend to the primary cache; the coupling vectors
a (query), b (MLP intermediate) and c (MLP output) carry primary values into
the auxiliary row only.

Layer form (readings where the pages are silent): pre-norm decoder block with
RMSNorm (shared gains, eps), fused Wqkv projection without bias and without a
positional rotation, grouped-query attention, output projection Wo, SwiGLU MLP
(silu(h Wg^T) * (h Wu^T)) Wd^T, fp32/fp64 residual streams. bf16 rounding
happens exactly at R1 (normed rows), R2 (appended K/V), R3 (attention output
entering Wo), R4 (normed rows), R5 (MLP intermediate entering Wd).
"""
import numpy as np

from .attention import decode_attention
from .cache import kv_append
from .linear import grouped_linear, rmsnorm, swiglu_couple
from .numerics import bf16_bits


def dual_flow_layer(x, g_attn, g_mlp, w_qkv, w_o, w_gate_up, w_down, a, b, c, eps,
                    k_pool, v_pool, block_table, context_lens_before, num_q_heads,
                    num_kv_heads, head_dim, batches=None, dtype=np.float64):
    """x: float [F][B][hidden] (F = 1 primary only, F = 2 both flows).

    context_lens_before[b] tokens are in the cache before the step; the
    primary row is appended at that position and both flows attend to
    context_lens_before[b] + 1 positions. Returns (x_out [F][B][hidden] fp64,
    k_pool', v_pool', dict of intermediates). ``batches`` limits attention to
    some sequences (their rows only are meaningful in x_out). ``dtype`` is the working
    precision: float64, or float32 for the same definition in single precision (whose
    distance from the float64 result measures how much the five bf16 rounding points
    amplify single-precision arithmetic).
    """
    x = np.asarray(x, dtype=np.float64)
    F, B, H = x.shape
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    h1 = rmsnorm(x, g_attn, eps, dtype)                            # R1
    qkv = grouped_linear(h1, w_qkv, dtype=dtype)
    q = qkv[..., : Hq * D]
    k_new = qkv[0, :, Hq * D: (Hq + Hkv) * D]
    v_new = qkv[0, :, (Hq + Hkv) * D:]
    pos = np.asarray(context_lens_before, dtype=np.int64)
    kp, vp = kv_append(k_pool, v_pool, block_table, pos, bf16_bits(k_new), bf16_bits(v_new))  # R2
    ctx = pos + 1
    o1, o2, _ = decode_attention(q[0].reshape(B, Hq, D), q[1].reshape(B, Hq, D) if F == 2 else None,
                                 a if F == 2 else None, 0, kp, vp, block_table, ctx, batches=batches,
                                 dtype=dtype)
    o = np.stack([o1] + ([o2] if F == 2 else [])).reshape(F, B, Hq * D)
    x1 = grouped_linear(o, w_o, residual=x, dtype=dtype)           # R3 inside (-> bf16)
    h2 = rmsnorm(x1, g_mlp, eps, dtype)                            # R4
    gu = grouped_linear(h2, w_gate_up, dtype=dtype)
    inter = swiglu_couple(gu, b if F == 2 else None, dtype)        # R5
    x2 = grouped_linear(inter, w_down, couple=c if F == 2 else None, residual=x1, dtype=dtype)
    return x2, kp, vp, dict(h1=h1, qkv=qkv, o=o, x1=x1, h2=h2, gu=gu, inter=inter)
