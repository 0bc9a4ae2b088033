"""Backward pass of the W4A16 linear with LoRA — oracle (test infrastructure only).

What it follows: QeRL explainer (lifetechia), "NVFP4 quantization and
LoRA" and "How QeRL combines quantization and LoRA": the base weights stay
frozen in NVFP4 and only the low-rank matrices are trained, so the backward
of the fused forward

    y = x deq(Wq)^T + s * (x A^T) B^T

needs the input gradient and the two adapter gradients, never a weight
gradient of the base:

    dX = dY deq(Wq) + s * (dY B) A        bf16 [M, K]
    dA = s * (dY B)^T x                   fp32 [r, K]
    dB = s * dY^T (x A^T)                 fp32 [N, r]

with dY bf16 [M, N]. These are plain definitions (the chain rule applied to
a sum of matrix products), so the oracle computes them directly: exact
widening of every bf16 operand and of the dequantised weight to float64,
float64 matmuls, one rounding at the end. Readings taken: dX is rounded once
to bf16 (nearest-even), the adapter gradients once to fp32; the pages fix
neither precision.

Pins (tests/test_oracle_lora_backward.py): exact Fraction evaluation on tiny
shapes (also of ``adapter_terms_f64``, the weight-free form used for sampled
checks at full size); the adjoint identities <dY, y(x + d) - y(x)> = <dX, d>, and the same
for A and B, against the forward oracle (y is linear in x and in each
adapter separately); r = 0 leaves only the base term; a zero weight leaves
only the LoRA terms.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, bf16_to_f64
from .nvfp4 import dequantize


def lora_linear_backward_f64(dy_bits, x_bits, codes, scales, s_t, a_bits=None, b_bits=None,
                             lora_scale: float = 0.0):
    """Unrounded (dX, dA, dB) in float64; dA and dB are None without adapters."""
    dy = bf16_to_f64(dy_bits)
    x = bf16_to_f64(x_bits)
    w = dequantize(codes, scales, s_t)  # [N, K], the frozen base
    dx = dy @ w
    if a_bits is None or b_bits is None or np.asarray(a_bits).shape[0] == 0:
        return dx, None, None
    a = bf16_to_f64(a_bits)   # [r, K]
    b = bf16_to_f64(b_bits)   # [N, r]
    s = np.float64(np.float32(lora_scale))
    g = dy @ b                # [M, r]: gradient reaching the rank space
    u = x @ a.T               # [M, r]: the down-projection of the forward
    dx = dx + s * (g @ a)
    da = s * (g.T @ x)
    db = s * (dy.T @ u)
    return dx, da, db


def backward_magnitudes_f64(dy_bits, x_bits, codes, scales, s_t, a_bits=None, b_bits=None,
                            lora_scale: float = 0.0):
    """The backward's sums with every term made non-negative (test tolerances only).

    Returns (dx_base, dx_lora, da, db): sum_n |dY||W|, sum_j |h_j| |A_jk| with
    |h| = |s| |dY| |B|, and the magnitudes of dA and dB; the last three are None
    without adapters. They bound the rounding error of any summation order.
    """
    dy = np.abs(bf16_to_f64(dy_bits))
    x = np.abs(bf16_to_f64(x_bits))
    dx_base = dy @ np.abs(dequantize(codes, scales, s_t))
    if a_bits is None or b_bits is None or np.asarray(a_bits).shape[0] == 0:
        return dx_base, None, None, None
    a = np.abs(bf16_to_f64(a_bits))
    b = np.abs(bf16_to_f64(b_bits))
    s = abs(np.float64(np.float32(lora_scale)))
    h = s * (dy @ b)
    u = x @ a.T
    return dx_base, h @ a, h.T @ x, s * (dy.T @ u)


def lora_linear_backward(dy_bits, x_bits, codes, scales, s_t, a_bits=None, b_bits=None,
                         lora_scale: float = 0.0):
    """(dX bf16-rounded, dA fp32-rounded, dB fp32-rounded), all as float64 arrays."""
    dx, da, db = lora_linear_backward_f64(dy_bits, x_bits, codes, scales, s_t, a_bits, b_bits,
                                          lora_scale)
    f32 = (lambda v: None if v is None else v.astype(np.float32).astype(np.float64))
    return bf16_round(dx), f32(da), f32(db)


def adapter_terms_f64(dy_bits, x_bits, a_bits, b_bits, lora_scale: float, b_rows=None):
    """(h, dA, dB[b_rows]) in float64, without building the dequantised weight.

    h = s (dY B) [M, r] is the gradient that reaches the rank space (it also
    feeds dX's LoRA term); dA = h^T x [r, K]; dB = s dY^T (x A^T), only the
    output features ``b_rows`` (all when None). For checks at full size,
    where the [N, K] float64 weight of ``lora_linear_backward_f64`` would be
    needlessly large.
    """
    dy = bf16_to_f64(dy_bits)
    x = bf16_to_f64(x_bits)
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    s = np.float64(np.float32(lora_scale))
    h = s * (dy @ b)
    da = h.T @ x
    u = x @ a.T
    dyr = dy if b_rows is None else dy[:, np.asarray(b_rows)]
    db = s * (dyr.T @ u)
    return h, da, db


def dx_columns_f64(dy_bits, codes, scales, s_t, cols, a_bits=None, h=None):
    """Unrounded dX[:, cols]; ``h`` = s (dY B) [M, r] in float64 when adapters are present.

    For sampled checks at full size: only the K columns ``cols`` of the
    dequantised weight are built.
    """
    from .nvfp4 import unpack_codes, code_value, e4m3_value, BLOCK

    cols = np.asarray(cols)
    c4 = unpack_codes(codes)[:, cols]
    g = np.asarray(code_value(c4), np.float64)
    sb = np.asarray(e4m3_value(np.asarray(scales)[:, cols // BLOCK]), np.float64)
    w = g * sb * np.float64(np.float32(s_t))
    dx = bf16_to_f64(dy_bits) @ w
    if h is not None and a_bits is not None:
        dx = dx + h @ bf16_to_f64(np.asarray(a_bits)[:, cols])
    return dx


def lora_backward_exact(dy_bits, x_bits, codes, scales, s_t, a_bits, b_bits, lora_scale):
    """(dX, dA, dB) as nested lists of Fractions, each term written out; tiny shapes only."""
    from fractions import Fraction as F
    from .nvfp4 import unpack_codes, code_value, e4m3_value, BLOCK

    dy = bf16_to_f64(dy_bits)
    x = bf16_to_f64(x_bits)
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    c4 = unpack_codes(codes)
    m, n = dy.shape
    k = x.shape[1]
    r = a.shape[0]
    st = F(float(np.float32(s_t)))
    s = F(float(np.float32(lora_scale)))
    w = [[F(float(code_value(c4[i, kk]))) * F(float(e4m3_value(scales[i, kk // BLOCK]))) * st
          for kk in range(k)] for i in range(n)]
    g = [[sum((F(float(dy[mm, i])) * F(float(b[i, j])) for i in range(n)), F(0)) for j in range(r)]
         for mm in range(m)]
    u = [[sum((F(float(x[mm, kk])) * F(float(a[j, kk])) for kk in range(k)), F(0)) for j in range(r)]
         for mm in range(m)]
    dx = [[sum((F(float(dy[mm, i])) * w[i][kk] for i in range(n)), F(0))
           + s * sum((g[mm][j] * F(float(a[j, kk])) for j in range(r)), F(0))
           for kk in range(k)] for mm in range(m)]
    da = [[s * sum((g[mm][j] * F(float(x[mm, kk])) for mm in range(m)), F(0)) for kk in range(k)]
          for j in range(r)]
    db = [[s * sum((F(float(dy[mm, i])) * u[mm][j] for mm in range(m)), F(0)) for j in range(r)]
          for i in range(n)]
    return dx, da, db
