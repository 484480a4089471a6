"""Grouped shared-weight linear, RMSNorm and SwiGLU with b-coupling (oracle, fp64).

Both flows apply the same attention, MLP and output matrices (Sintesi
Tecnica: Dual-Flow Transformers, "Architettura Core"), so one weight matrix
serves the rows of both flows. The auxiliary flow is enriched one way from
the primary through learned vectors at the MLP-intermediate (b) and
MLP-output (c) levels ("Meccanismi Chiave"); the pages give no formula, and
the reading used here is elementwise addition of the primary's value scaled
by the vector: inter_aux += b * inter_prim after the gated activation,
mlp_aux += c * mlp_prim before the residual add.
"""
import numpy as np

from .numerics import bf16_bits, round_bf16, widen


def grouped_linear(x, w, couple=None, residual=None, y_bf16=False, dtype=np.float64):
    """Y[f] = bf16(X[f]) @ W^T for every flow f, then the optional coupling
    Y[1] += couple * Y[0], then the optional residual add.

    x: [F][rows][K] (uint16 bf16 bits, or float32/float64 which are rounded to
    bf16 first); w: [N][K] uint16 bf16 bits. Returns float64 [F][rows][N], or
    bf16 bits when y_bf16. ``dtype`` is the working precision of the arithmetic (float64;
    float32 gives the same definition evaluated in single precision).
    """
    x = np.asarray(x)
    X = (widen(x) if x.dtype == np.uint16 else round_bf16(widen(x))).astype(dtype)
    W = widen(w).astype(dtype)
    Y = X @ W.T
    if couple is not None and Y.shape[0] == 2:
        Y[1] = Y[1] + widen(couple).astype(dtype) * Y[0]
    if residual is not None:
        Y = widen(residual).astype(dtype) + Y
    return bf16_bits(Y) if y_bf16 else Y


def rmsnorm(x, gain, eps, dtype=np.float64, rounded=True):
    """y = x / sqrt(mean(x^2) + eps) * gain over the last axis, rounded to bf16 (fp64 values);
    rounded=False returns the value before that rounding."""
    X = widen(x).astype(dtype)
    r = dtype(1.0) / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + dtype(eps))
    y = X * r * widen(gain).astype(dtype)
    return round_bf16(y) if rounded else y


def swiglu_couple(gate_up, b=None, dtype=np.float64, rounded=True):
    """inter = silu(gate) * up with gate_up = [gate | up] on the last axis; for
    two flows inter[1] += b * inter[0]; rounded to bf16 (fp64 values); rounded=False
    returns the value before that rounding."""
    GU = widen(gate_up).astype(dtype)
    I = GU.shape[-1] // 2
    gate, up = GU[..., :I], GU[..., I:]
    inter = gate / (dtype(1.0) + np.exp(-gate)) * up
    if b is not None and inter.shape[0] == 2:
        inter[1] = inter[1] + widen(b).astype(dtype) * inter[0]
    return round_bf16(inter) if rounded else inter
