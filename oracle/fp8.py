"""FP8 (E4M3) rollout linear, W8A16 with LoRA — oracle (test infrastructure only).

What it follows: the gist.science summary of adaptive importance sampling
for quantized RL ("Problem definition"; "Experimental results", efficiency):
rollout engines run the policy in low precision such as FP8 while the
trainer keeps BF16, and FP8 rollout halves the rollout model's footprint.
The page fixes no FP8 layout or scaling. Readings taken:

* weights are OCP E4M3 (e4m3fn: bias 7, max 448, subnormals m 2^-9), one
  fp32 scale per output row, s_n = fp32(amax_n / 448) (s_n = 0 for an
  all-zero row, whose codes are all 0);
* the code of w[n, k] is the nearest finite E4M3 value to the fp32 quotient
  fp32(w / s_n), ties to the even mantissa, saturating at 448; the sign bit
  is set when w < 0 and the magnitude code is not zero (so no -0 codes);
* activations stay bf16 (W8A16), and the LoRA update is the one of the
  NVFP4 linear: y = bf16(x deq(W8)^T + s (x A^T) B^T), deq = e4m3 * s_n.

The quantiser's rounding takes the nearest-value definition (``e4m3_encode``
of the NVFP4 oracle, pinned against torch's float8 cast); the linear is a
plain definition, computed in float64 with one rounding to bf16.

Pins (tests/test_oracle_fp8.py): torch's CPU float8_e4m3fn cast of the same
fp32 quotients; the row amax element maps to 448 (byte 0x7E); the error
bound |w - deq| <= half an E4M3 step * s_n; sign symmetry; exact Fraction
evaluation of the linear on tiny shapes. W8A8 (below): exact Fractions over
decoded bytes; equality with W8A16 when every token row already lies on a
power-of-two-scaled E4M3 grid; the activation-error bound against W8A16.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, bf16_to_f64
from .nvfp4 import E4M3_MAX, e4m3_encode, e4m3_value


def row_scales(w) -> np.ndarray:
    """s_n = fp32(amax_n / 448), fp32 [N]."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1) if w.shape[1] else np.zeros(w.shape[0], np.float32)
    return (amax.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)


def quantize(w) -> tuple[np.ndarray, np.ndarray]:
    """(codes u8 [N, K], row scales fp32 [N])."""
    w = np.asarray(w, dtype=np.float32)
    s = row_scales(w)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[:, None] > 0, w / np.where(s > 0, s, np.float32(1))[:, None], np.float32(0))
    q = q.astype(np.float32)  # the fp32 quotient decides the code
    mag = e4m3_encode(np.abs(q).astype(np.float64))
    sign = (q < 0) & (mag != 0)
    return (mag | np.where(sign, 0x80, 0)).astype(np.uint8), s


def dequantize(codes, s) -> np.ndarray:
    """W[n, k] = +-e4m3(code) * s_n, exact in float64."""
    c = np.asarray(codes, dtype=np.uint8)
    v = e4m3_value(c & 0x7F).astype(np.float64)
    v = np.where(c & 0x80, -v, v)
    return v * np.asarray(s, dtype=np.float32).astype(np.float64)[:, None]


def lora_linear_f64(x_bits, codes, s, a_bits=None, b_bits=None, lora_scale: float = 0.0) -> np.ndarray:
    x = bf16_to_f64(x_bits)
    y = x @ dequantize(codes, s).T
    if a_bits is not None and b_bits is not None and np.asarray(a_bits).shape[0] > 0:
        t = x @ bf16_to_f64(a_bits).T
        y = y + np.float64(np.float32(lora_scale)) * (t @ bf16_to_f64(b_bits).T)
    return y


def lora_linear(x_bits, codes, s, a_bits=None, b_bits=None, lora_scale: float = 0.0) -> np.ndarray:
    """bf16-rounded y [M, N] (float64 values)."""
    return bf16_round(lora_linear_f64(x_bits, codes, s, a_bits, b_bits, lora_scale))


def lora_linear_exact(x_bits, codes, s, a_bits, b_bits, lora_scale):
    """The same sum in Fractions, every term written out; tiny shapes only."""
    from fractions import Fraction as F

    x = bf16_to_f64(x_bits)
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    m, k = x.shape
    n, r = b.shape
    sc = F(float(np.float32(lora_scale)))
    out = [[None] * n for _ in range(m)]
    for i in range(m):
        t = [sum((F(float(x[i, kk])) * F(float(a[j, kk])) for kk in range(k)), F(0)) for j in range(r)]
        for nn in range(n):
            acc = F(0)
            for kk in range(k):
                c = int(codes[nn, kk])
                v = F(float(e4m3_value(c & 0x7F))) * (-1 if c & 0x80 else 1)
                acc += F(float(x[i, kk])) * v * F(float(np.float32(s[nn])))
            out[i][nn] = acc + sc * sum((t[j] * F(float(b[nn, j])) for j in range(r)), F(0))
    return out


# --- W8A8: activations quantised too -------------------------------------
#
# The pages name FP8 rollout without saying whether activations are
# quantised; the W8A8 reading taken here is the plainest one that matches
# the weight recipe above:
#
# * each token (row m of x) gets one fp32 scale s_x[m] = fp32(amax_m / 448)
#   and E4M3 codes by the same nearest-value encoder as the weights, applied
#   to the fp32 quotient fp32(x / s_x[m]) of the bf16 input widened to fp32;
# * the base product is the exact sum of decoded codes,
#   y_base[m, n] = s_x[m] * s_n * sum_k e4m3(x8[m, k]) * e4m3(w8[n, k]);
# * the LoRA branch reads the unquantised bf16 x, as in W8A16 (only the
#   frozen base weight's product runs in FP8);
# * y = bf16(y_base + s (x A^T) B^T), one rounding.


def quantize_activations(x_bits) -> tuple[np.ndarray, np.ndarray]:
    """Per-token E4M3 codes u8 [M, K] and scales fp32 [M] of bf16 x."""
    return quantize(bf16_to_f64(x_bits).astype(np.float32))


def w8a8_lora_linear_f64(x_bits, codes, s, a_bits=None, b_bits=None, lora_scale: float = 0.0) -> np.ndarray:
    x8, sx = quantize_activations(x_bits)
    y = dequantize(x8, sx) @ dequantize(codes, s).T
    if a_bits is not None and b_bits is not None and np.asarray(a_bits).shape[0] > 0:
        x = bf16_to_f64(x_bits)
        t = x @ bf16_to_f64(a_bits).T
        y = y + np.float64(np.float32(lora_scale)) * (t @ bf16_to_f64(b_bits).T)
    return y


def w8a8_lora_linear(x_bits, codes, s, a_bits=None, b_bits=None, lora_scale: float = 0.0) -> np.ndarray:
    """bf16-rounded W8A8 y [M, N] (float64 values)."""
    return bf16_round(w8a8_lora_linear_f64(x_bits, codes, s, a_bits, b_bits, lora_scale))


def w8a8_magnitude_f64(x_bits, codes, s, a_bits=None, b_bits=None, lora_scale: float = 0.0):
    """(base, lora) sums of |terms| of the W8A8 product, for accumulation-error bounds."""
    x8, sx = quantize_activations(x_bits)
    base = np.abs(dequantize(x8, sx)) @ np.abs(dequantize(codes, s)).T
    lora = np.zeros_like(base)
    if a_bits is not None and b_bits is not None and np.asarray(a_bits).shape[0] > 0:
        x = np.abs(bf16_to_f64(x_bits))
        t = x @ np.abs(bf16_to_f64(a_bits)).T
        lora = abs(float(np.float32(lora_scale))) * (t @ np.abs(bf16_to_f64(b_bits)).T)
    return base, lora


def w8a8_lora_linear_exact(x_bits, codes, s, a_bits, b_bits, lora_scale):
    """The W8A8 sum in Fractions over decoded bytes of both operands; tiny shapes only."""
    from fractions import Fraction as F

    x8, sx = quantize_activations(x_bits)
    x = bf16_to_f64(x_bits)
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    m, k = x.shape
    n, r = b.shape
    sc = F(float(np.float32(lora_scale)))

    def dec(c):
        c = int(c)
        return F(float(e4m3_value(c & 0x7F))) * (-1 if c & 0x80 else 1)

    out = [[None] * n for _ in range(m)]
    for i in range(m):
        t = [sum((F(float(x[i, kk])) * F(float(a[j, kk])) for kk in range(k)), F(0)) for j in range(r)]
        for nn in range(n):
            acc = sum((dec(x8[i, kk]) * dec(codes[nn, kk]) for kk in range(k)), F(0))
            acc *= F(float(np.float32(sx[i]))) * F(float(np.float32(s[nn])))
            out[i][nn] = acc + sc * sum((t[j] * F(float(b[nn, j])) for j in range(r)), F(0))
    return out
