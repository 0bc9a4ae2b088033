"""W4A16 linear with the LoRA update — oracle (test infrastructure only).

What it follows: QeRL explainer (lifetechia), "NVFP4 quantization and
LoRA" and "How QeRL combines quantization and LoRA": the base weights are
frozen in NVFP4, training adds trainable low-rank matrices, and rollout runs
the quantised base with 16-bit activations ("NVFP4 + Marlin kernel",
section "Experimental details"). The fused forward is

    y = x deq(Wq)^T + s * (x A^T) B^T

with x bf16 [M, K], Wq NVFP4 [N, K], A bf16 [r, K], B bf16 [N, r], s fp32.

This is a plain definition, so the oracle computes it directly: dequantise W
exactly (float64), widen the bf16 operands exactly, two float64 matmuls, and
one rounding of the result to bf16 (nearest-even). Reading taken: the output
is bf16 and the LoRA product is kept unrounded (float64) before the sum.

Pins (tests/test_oracle_linear.py): exact Fraction evaluation of the sum on
tiny shapes; B = 0 and s = 0 reduce to the base product; W = 0 reduces to
the LoRA product; y(2x) = 2 y(x) exactly. The down-projection t = s x A^T
on its own (``lora_down``) is pinned term by term against Fractions on
non-square adapters, at two scales, so a dropped s or a transposed A fails.
The magnitude sums (``lora_linear_magnitude_f64``, test tolerances only)
equal the linear itself on non-negative inputs and bound its absolute value
everywhere.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, bf16_to_f64
from .nvfp4 import dequantize, unpack_codes, code_value, e4m3_value, BLOCK


def lora_linear_f64(x_bits, codes, scales, s_t, a_bits=None, b_bits=None,
                    lora_scale: float = 0.0, rows=None) -> np.ndarray:
    """Unrounded y (float64) of the fused linear; ``rows`` selects output columns n."""
    x = bf16_to_f64(x_bits)
    if rows is not None:
        rows = np.asarray(rows)
        codes = np.asarray(codes)[rows]
        scales = np.asarray(scales)[rows]
        if b_bits is not None:
            b_bits = np.asarray(b_bits)[rows]
    w = dequantize(codes, scales, s_t)
    y = x @ w.T
    if a_bits is not None and b_bits is not None and np.asarray(a_bits).shape[0] > 0:
        a = bf16_to_f64(a_bits)
        b = bf16_to_f64(b_bits)
        t = x @ a.T
        y = y + np.float64(np.float32(lora_scale)) * (t @ b.T)
    return y


def lora_linear(x_bits, codes, scales, s_t, a_bits=None, b_bits=None,
                lora_scale: float = 0.0, rows=None) -> np.ndarray:
    """bf16-rounded y [M, N] (float64 values), the device output's reference."""
    return bf16_round(lora_linear_f64(x_bits, codes, scales, s_t, a_bits, b_bits,
                                      lora_scale, rows))


def lora_linear_magnitude_f64(x_bits, codes, scales, s_t, a_bits=None, b_bits=None,
                              lora_scale: float = 0.0, rows=None):
    """(base, lora): sum_k |x_k| |W_nk| and |s| sum_j (sum_k |x_k| |A_jk|) |B_nj|, float64 [M, N].

    The same sums as the linear with every term made non-negative: they bound
    the rounding error of any order of summation, so tests derive their
    per-element tolerances from them. ``rows`` selects output features as in
    ``lora_linear_f64``.
    """
    x = np.abs(bf16_to_f64(x_bits))
    if rows is not None:
        rows = np.asarray(rows)
        codes = np.asarray(codes)[rows]
        scales = np.asarray(scales)[rows]
        if b_bits is not None:
            b_bits = np.asarray(b_bits)[rows]
    base = x @ np.abs(dequantize(codes, scales, s_t)).T
    lora = np.zeros_like(base)
    if a_bits is not None and b_bits is not None and np.asarray(a_bits).shape[0] > 0:
        t = x @ np.abs(bf16_to_f64(a_bits)).T
        lora = abs(np.float64(np.float32(lora_scale))) * (t @ np.abs(bf16_to_f64(b_bits)).T)
    return base, lora


def lora_down(x_bits, a_bits, lora_scale: float) -> np.ndarray:
    """t = s * x A^T, float64 [M, r] (the LoRA down-projection, unrounded).

    x bf16 [M, K] and A bf16 [r, K] as in the fused formula; s is taken at
    fp32 precision, the precision the library receives it in.
    """
    return np.float64(np.float32(lora_scale)) * (bf16_to_f64(x_bits) @ bf16_to_f64(a_bits).T)


def lora_down_exact(x_bits, a_bits, lora_scale: float):
    """The same t as nested lists of Fractions, every product written out; tiny shapes only."""
    from fractions import Fraction as F

    x = bf16_to_f64(x_bits)
    a = bf16_to_f64(a_bits)
    s = F(float(np.float32(lora_scale)))
    m, k = x.shape
    r = a.shape[0]
    return [[s * sum((F(float(x[i, kk])) * F(float(a[j, kk])) for kk in range(k)), F(0))
             for j in range(r)] for i in range(m)]


def lora_linear_exact(x_bits, codes, scales, s_t, a_bits, b_bits, lora_scale):
    """Same sum in exact rational arithmetic (Fractions); tiny shapes only.

    Used to pin the float64 path: every term is written out one by one, with
    the dequantised weight rebuilt from the code nibble, the E4M3 byte and s_t.
    """
    from fractions import Fraction as F

    x = bf16_to_f64(x_bits)
    c4 = unpack_codes(codes)
    m, k = x.shape
    n = c4.shape[0]
    r = 0 if a_bits is None else np.asarray(a_bits).shape[0]
    a = bf16_to_f64(a_bits) if r else None
    b = bf16_to_f64(b_bits) if r else None
    st = F(float(np.float32(s_t)))
    s = F(float(np.float32(lora_scale)))
    out = [[None] * n for _ in range(m)]
    for i in range(m):
        t = [sum((F(float(x[i, kk])) * F(float(a[j, kk])) for kk in range(k)), F(0))
             for j in range(r)]
        for nn in range(n):
            acc = F(0)
            for kk in range(k):
                g = F(float(code_value(c4[nn, kk])))
                sb = F(float(e4m3_value(scales[nn, kk // BLOCK])))
                acc += F(float(x[i, kk])) * g * sb * st
            for j in range(r):
                acc += s * t[j] * F(float(b[nn, j]))
            out[i][nn] = acc
    return out
