"""bf16 codec of the oracle (test infrastructure only).

bf16 is 1 sign bit, 8 exponent bits and 7 stored significand bits: the upper half
of an IEEE binary32. Rounding here is the plain definition: the nearest bf16 value,
ties to the one with an even last significand bit, applied directly to the float64
value (no intermediate float32 rounding). Signed zeros survive underflow, values at
or beyond the overflow midpoint become infinities, NaN becomes the quiet NaN 0x7FC0.

The TensorFold pull request #1186 ("cuda gemma4: images on the 31B", commit message
on bf16 rounding of tiny negatives) states the edge cases this must honour:
bf16(-2^-135) is -0 (0x8000), with signed zeros from underflow, subnormal ties, the
normal boundary and overflow to both infinities compared as u16 bits.
"""
from __future__ import annotations

import numpy as np

_MIN_EXP = -133  # bf16 subnormal quantum is 2^-133 (2^-126 with 7 fraction bits)
_OVERFLOW = 2.0 ** 128  # anything that rounds to 2^128 or beyond is infinite


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) and return uint16 bits."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        # ax = f * 2^e2 with f in [0.5, 1): the leading bit has weight 2^(e2 - 1).
        _, e2 = np.frexp(ax)
        lead = e2.astype(np.int64) - 1
        # 8 significant bits for normals; a fixed 2^-133 quantum below 2^-126.
        quantum_exp = np.maximum(lead - 7, _MIN_EXP).astype(np.int32)
        q = np.ldexp(1.0, quantum_exp)
        r = np.round(ax / q) * q  # exact scaling; np.round is half-to-even
        r = np.where(np.isinf(ax), np.inf, r)
        r = np.where(r >= _OVERFLOW, np.inf, r)
        signed = np.copysign(r, x)
        out = (signed.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out = np.where(np.isnan(x), np.uint16(0x7FC0), out)
    return out.astype(np.uint16)


def round_f64(x) -> np.ndarray:
    """float64 -> nearest bf16 -> float64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))
