"""Rounding helpers of the oracle (test infrastructure only).

bf16 is the 16-bit float with fp32's 8-bit exponent and 7 stored mantissa
bits. Outputs of the linear and of the RMSNorm are bf16, so the oracle rounds
its exact (float64) results to bf16 once, to nearest with ties to even, and
compares against the device's bf16 outputs.

Pinned by tests/test_oracle_numerics.py against torch's CPU float32->bf16
cast (exhaustive over sampled float32 patterns) and against exact Fraction
rounding for float64 inputs.
"""
from __future__ import annotations

import numpy as np

_BF16_MIN_EXP = -126      # smallest normal exponent (same as fp32)
_BF16_MANT = 7            # stored mantissa bits
_BF16_MAX = float.fromhex("0x1.fep127")


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    Single rounding straight from float64. Values whose magnitude rounds past
    the largest finite bf16 become +-inf, as IEEE rounding does. Subnormal
    bf16 values (quantum 2^-133) are kept.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    finite = np.isfinite(v)
    out[~finite] = v[~finite]
    f = v[finite]
    a = np.abs(f)
    # exponent e with 2^e <= |v| < 2^(e+1); quantum = 2^(max(e, -126) - 7)
    _, e2 = np.frexp(a)                 # a = m * 2^e2, m in [0.5, 1)
    e = e2.astype(np.int64) - 1
    e = np.maximum(e, _BF16_MIN_EXP)
    q_exp = e - _BF16_MANT
    scaled = np.ldexp(f, -q_exp)        # exact: power-of-two scaling
    r = np.rint(scaled)                 # numpy rint: round half to even
    res = np.ldexp(r, q_exp)
    res = np.where(np.abs(res) > _BF16_MAX, np.copysign(np.inf, f), res)
    out[finite] = res
    return out


def bf16_bits_of(values) -> np.ndarray:
    """bf16 bit pattern (uint16) of values that are already exact bf16 numbers."""
    f32 = np.asarray(values, dtype=np.float64).astype(np.float32)
    bits = f32.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not exact bf16 numbers")
    return (bits >> 16).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rel_l2(y, y_ref) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 over the whole tensor, in float64."""
    y = np.asarray(y, dtype=np.float64).ravel()
    r = np.asarray(y_ref, dtype=np.float64).ravel()
    den = np.linalg.norm(r)
    num = np.linalg.norm(y - r)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
