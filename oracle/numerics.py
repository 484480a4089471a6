"""Exact widening of stored inputs and direct fp64 -> bf16 rounding (oracle only).

bf16 keeps fp32's 8-bit exponent and 8 significant bits. Widening a bf16 bit
pattern is a 16-bit left shift into an fp32 pattern, exact in fp64. Rounding
an fp64 value to bf16 is done here in one step (not through fp32), round to
nearest, ties to even, as IEEE 754 defines it for a narrower format.
"""
import numpy as np

BF16_MAX = float.fromhex("0x1.fe00000000000p+127")   # largest finite bf16
_MIN_EXP_QUANTUM = 2.0 ** -133                       # spacing of bf16 subnormals


def widen(x) -> np.ndarray:
    """uint16 (bf16 bits) / float32 / float64 array -> float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even); result as fp64.

    For |x| in [2^(e-1), 2^e) the bf16 spacing is 2^(e-8); below the normal
    range the spacing is fixed at 2^-133. Scaling by a power of two is exact,
    and np.rint rounds half to even, so the rounded value is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)
    q = np.maximum(np.ldexp(1.0, e - 8), _MIN_EXP_QUANTUM)
    y = np.rint(xf / q) * q
    y[np.abs(y) > BF16_MAX] = np.copysign(np.inf, y[np.abs(y) > BF16_MAX])
    out[fin] = y
    return out


def bf16_bits(x) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16) after round_bf16; NaN -> 0x7FC0."""
    y = round_bf16(x)
    bits = (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(y)] = 0x7FC0
    return bits
