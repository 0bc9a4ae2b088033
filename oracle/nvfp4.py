"""NVFP4 block quantiser and dequantiser — oracle (test infrastructure only).

What it follows:

* QeRL explainer (lifetechia), "NVFP4 quantization and LoRA": the frozen
  base weights are held in 4-bit NVFP4.
* TRACE article (sns.style), "Engineering view of the mechanism": FP4 uses
  block scaling, a small group of values shares one scale, and each value is
  rounded up or down to a neighbouring point of the 4-bit grid — a discrete
  per-value choice.
* The NVFP4 format itself: 16-element blocks along the reduction dim, one
  E4M3 (OCP e4m3fn) scale per block, one FP32 scale per tensor, element codes
  on the E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit.

The pages fix neither the scale recipe nor the rounding mode; the readings
taken here are:

1. s_t = fp32(amax / 2688), 2688 = 6 * 448 (largest E2M1 x largest E4M3).
2. block byte = E4M3 nearest-even, saturating at 448, of
   r_b = fp32(a_b / fp32(6 * s_t)); a zero block or s_t == 0 gives byte 0.
3. D_b = fp32(S_b * s_t); each element goes to the E2M1 grid point g_k * D_b
   nearest to |x| in exact arithmetic, ties to the even index k (IEEE
   round-half-even on the E2M1 mantissa); the sign bit is the sign of x
   (so -0.0 and tiny negatives give code 0x8); D_b == 0 gives magnitude 0.
4. Layout: codes [N][K/2] bytes, element 2j in the low nibble of byte j;
   scales [N][K/16] bytes; both row-major, blocks along K.

Pins (tests/test_oracle_nvfp4.py): Fraction brute force over all 16 codes on
tiny blocks; exhaustive E4M3 check against torch's CPU float8_e4m3fn cast;
hand-worked golden blocks (tests/golden/nvfp4_blocks.txt); the per-element
error bound; power-of-two / sign / permutation equivariances.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
TENSOR_DIVISOR = np.float32(E2M1_MAX * E4M3_MAX)   # 2688


def e4m3_value(byte) -> np.ndarray:
    """Value of OCP E4M3FN bytes (bias 7, no infinities, 0x7F/0xFF = NaN)."""
    b = np.asarray(byte, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return sign * val


# the 127 finite non-negative E4M3 values, by byte 0x00..0x7E (increasing)
_E4M3_POS = e4m3_value(np.arange(0x7F))


def e4m3_encode(r) -> np.ndarray:
    """Nearest finite non-negative E4M3 byte to r (>= 0), ties to the even byte.

    Bytes 0x00..0x7E are increasing in value, and an even byte is an even
    mantissa, so "nearest, ties to even byte" is IEEE round-half-even; taking
    the nearest *finite* value is the saturating (satfinite) variant: every
    r >= 448 maps to 0x7E. Subnormals (m * 2^-9) are kept.
    """
    r = np.asarray(r, dtype=np.float64)
    if np.any(~np.isfinite(r)) or np.any(r < 0):
        raise ValueError("e4m3_encode expects finite non-negative input")
    lo = np.clip(np.searchsorted(_E4M3_POS, r, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = r - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - r
    # differences are exact: r and the table values are float32 numbers within
    # a factor of two of each other (or r beyond the table, where hi == lo)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    return np.where(pick_hi, hi, lo).astype(np.uint8)


def tensor_scale(w: np.ndarray) -> np.float32:
    """s_t = fp32(amax / 2688); amax = max |W| (exact). Non-finite input -> error."""
    w = np.asarray(w, dtype=np.float32)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    if w.size == 0:
        return np.float32(0.0)
    amax = np.float32(np.max(np.abs(w)))
    return np.float32(amax / TENSOR_DIVISOR)


def block_scale_bytes(w: np.ndarray, s_t: np.float32) -> np.ndarray:
    """E4M3 scale byte of every 16-element block of W [N, K]."""
    n, k = w.shape
    blocks = np.abs(w.astype(np.float32)).reshape(n, k // BLOCK, BLOCK)
    a_b = blocks.max(axis=2)
    if s_t == 0:
        return np.zeros((n, k // BLOCK), dtype=np.uint8)
    six_st = np.float32(np.float32(6.0) * np.float32(s_t))
    r_b = (a_b / six_st).astype(np.float32)          # fp32 division, RNE
    return e4m3_encode(r_b)


def e2m1_index(ax: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Index k of the E2M1 magnitude g_k with g_k * d nearest to ax, ties to even k.

    ax, d: float64 arrays holding float32 values (ax >= 0, d >= 0). The grid
    points g_k*d are consecutive; |x| goes to g_k*d exactly when it lies
    between the midpoints (g_{k-1}+g_k)/2*d and (g_k+g_{k+1})/2*d. Each
    midpoint times d has at most 27 significant bits, so the float64 products
    and comparisons below are exact. On a tie the even k wins: midpoints
    0.25, 1.25, 2.5, 5 fall toward the lower (even) index, 0.75, 1.75, 3.5
    toward the upper (even) one. d == 0 gives index 0.
    """
    mids = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2.0     # 0.25 .. 5
    k = np.zeros(ax.shape, dtype=np.int64)
    for j, mj in enumerate(mids):
        edge = mj * d
        upper_even = (j + 1) % 2 == 0                  # tie goes to index j+1
        k += (ax > edge) | (upper_even & (ax == edge))
    return np.where(d == 0, 0, k)


def quantize(w) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """NVFP4-quantise W [N, K] (fp32 values; bf16 inputs widen exactly).

    Returns (codes uint8 [N, K/2], scales uint8 [N, K/16], s_t float32).
    Steps in order: tensor amax -> s_t -> per-block E4M3 scale byte ->
    D_b = fp32(S_b * s_t) -> per-element nearest E2M1 code -> nibble packing.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("W must be [N, K] with K a multiple of 16")
    n, k = w.shape
    s_t = tensor_scale(w)
    sbytes = block_scale_bytes(w, s_t)
    s_b = e4m3_value(sbytes).astype(np.float32)
    d_b = (s_b * s_t).astype(np.float32)             # fp32 product, RNE
    d_el = np.repeat(d_b.astype(np.float64), BLOCK, axis=1)
    ax = np.abs(w).astype(np.float64)
    idx = e2m1_index(ax, d_el)
    sign = np.signbit(w).astype(np.int64)
    codes4 = (sign << 3) | idx
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbytes, s_t


def quantize_rows(w, rows) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """``quantize`` restricted to the given rows of W (s_t still from all of W).

    Blocks never cross rows, so each row's codes and scale bytes depend only on
    that row and the tensor scale; this is the same definition evaluated on a
    sample, for matrices too large to encode whole on the CPU.
    """
    w = np.asarray(w, dtype=np.float32)
    s_t = tensor_scale(w)
    sub = w[np.asarray(rows)]
    sbytes = block_scale_bytes(sub, s_t)
    s_b = e4m3_value(sbytes).astype(np.float32)
    d_b = (s_b * s_t).astype(np.float32)
    d_el = np.repeat(d_b.astype(np.float64), BLOCK, axis=1)
    idx = e2m1_index(np.abs(sub).astype(np.float64), d_el)
    codes4 = (np.signbit(sub).astype(np.int64) << 3) | idx
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbytes, s_t


def rounding_record(w) -> np.ndarray:
    """Per-element rounding direction of ``quantize(w)``: uint8 [N, K/8] bit mask.

    TRACE article (sns.style), "Engineering view of the mechanism": under
    block scaling every value is rounded up or down to a neighbouring grid
    point, a discrete per-value choice, and the rollout side records its
    quantisation so that the trainer can reproduce it ("TRACE's core idea":
    rollout-guided rounding, with a compact cache of that information). The
    pages do not fix the record's format; the reading taken here is one bit
    per element: 1 when the magnitude was rounded up, i.e. the chosen grid
    point g_k * D_b (D_b = fp32(S_b * s_t), the grid the codes were chosen
    on) exceeds |x|; 0 when it was rounded down or hit exactly, and for blocks
    with D_b == 0. Bit e of byte j holds element 8 j + e of the row. Together
    with the scale bytes this is the record the trainer needs: the rounding
    of x is floor or ceil on the grid, and the bit says which.

    g_k has at most 2 significant bits and D_b at most 24, so the float64
    product and the comparison are exact.
    """
    w = np.asarray(w, dtype=np.float32)
    packed, sbytes, s_t = quantize(w)
    s_b = e4m3_value(sbytes).astype(np.float32)
    d_b = (s_b * s_t).astype(np.float32)
    d_el = np.repeat(d_b.astype(np.float64), BLOCK, axis=1)
    g = E2M1_GRID[unpack_codes(packed) & 7]
    up = (g * d_el > np.abs(w).astype(np.float64)).astype(np.uint8)
    n, k = w.shape
    bits = up.reshape(n, k // 8, 8) << np.arange(8, dtype=np.uint8)
    return bits.sum(axis=2).astype(np.uint8)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[N, K/2] packed bytes -> [N, K] 4-bit codes (element 2j = low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


def code_value(code4) -> np.ndarray:
    """Signed E2M1 value of 4-bit codes: bit 3 is the sign, bits 0-2 index the grid."""
    c = np.asarray(code4, dtype=np.int64)
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def dequantize(codes, scales, s_t) -> np.ndarray:
    """W_hat[n,k] = g(code) * S_b * s_t, exact in float64 (<= 30 significant bits)."""
    c4 = unpack_codes(codes)
    g = code_value(c4)
    s_b = np.repeat(e4m3_value(scales), BLOCK, axis=1)
    return g * s_b * np.float64(np.float32(s_t))
