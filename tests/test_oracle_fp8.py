"""Pins of the FP8 (E4M3) rollout oracle (CPU only)."""
import numpy as np
import torch

from oracle import fp8
from oracle.numerics import bf16_round
from oracle.nvfp4 import e4m3_value
from workloads import bf16_bits, lora_bf16, normal_f32


def test_codes_match_torch_float8_cast():
    """Codes of in-range quotients equal torch's CPU float8_e4m3fn cast (nearest, ties to even)."""
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 256)) * 10.0 ** rng.integers(-6, 3, (64, 256))).astype(np.float32)
    w[3] = 0.0
    codes, s = fp8.quantize(w)
    q = np.where(s[:, None] > 0, w / np.where(s > 0, s, 1)[:, None], 0).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = np.where((ref & 0x7F) == 0, 0, ref)  # the oracle writes no -0 codes
    assert np.array_equal(codes, ref)
    assert not codes[3].any() and s[3] == 0


def test_scale_and_amax_code():
    w = normal_f32((32, 96), 0.02, 2)
    codes, s = fp8.quantize(w)
    amax = np.max(np.abs(w), axis=1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # the element of largest magnitude lands on 448 (byte 0x7E with its sign)
    j = np.argmax(np.abs(w), axis=1)
    assert np.all(codes[np.arange(32), j] & 0x7F == 0x7E)


def test_error_bound_and_sign_symmetry():
    w = normal_f32((48, 160), 0.05, 3)
    codes, s = fp8.quantize(w)
    deq = fp8.dequantize(codes, s)
    # half the E4M3 step at the element's binade (normal: 2^(e-3); subnormal: 2^-9), times s_n
    q = np.abs(w.astype(np.float64)) / s[:, None].astype(np.float64)
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    half_step = 0.5 * 2.0 ** (e - 3)
    assert np.all(np.abs(w - deq) <= half_step * s[:, None] * (1 + 1e-6))
    c2, s2 = fp8.quantize(-w)
    assert np.array_equal(s, s2) and np.array_equal(c2 & 0x7F, codes & 0x7F)
    nz = (codes & 0x7F) != 0
    assert np.array_equal((c2 ^ codes)[nz], np.full(int(nz.sum()), 0x80, np.uint8))


def test_linear_matches_exact_rationals_and_reduces():
    rng = np.random.default_rng(4)
    for (m, n, k, r) in [(2, 3, 32, 2), (3, 2, 48, 1)]:
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        x = bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
        a, b = lora_bf16(r, k, n, m + n)
        codes, s = fp8.quantize(w)
        y = fp8.lora_linear_f64(x, codes, s, a, b, 2.0)
        ex = np.array([[float(v) for v in row] for row in fp8.lora_linear_exact(x, codes, s, a, b, 2.0)])
        assert np.allclose(y, ex, rtol=1e-13, atol=0)
        assert np.array_equal(bf16_round(y), bf16_round(ex))
    # B = 0: the base product alone, checked against plain sums of decoded bytes
    codes, s = fp8.quantize(w)
    base = fp8.lora_linear(x, codes, s)
    assert np.array_equal(fp8.lora_linear(x, codes, s, a, np.zeros_like(b), 2.0), base)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for i in range(m):
        for nn in range(n):
            want = sum(xv[i, kk] * float(e4m3_value(codes[nn, kk] & 0x7F)) * (-1 if codes[nn, kk] & 0x80 else 1)
                       for kk in range(k)) * float(s[nn])
            assert bf16_round(np.array([want]))[0] == base[i, nn]


def _grid_rows(rng, m, k, shifts):
    """bf16 token rows whose values already sit on 2^-j * E4M3, with amax = 448 * 2^-j."""
    mags = np.array([e4m3_value(c) for c in range(0x7F)], np.float64)
    x = np.empty((m, k), np.float64)
    for i in range(m):
        row = mags[rng.integers(0, 0x7F, k)] * rng.choice([-1.0, 1.0], k)
        row[rng.integers(0, k)] = 448.0 * rng.choice([-1.0, 1.0])
        x[i] = row * 2.0 ** -shifts[i % len(shifts)]
    return bf16_bits(x.astype(np.float32))


def test_w8a8_matches_exact_rationals():
    rng = np.random.default_rng(11)
    for (m, n, k, r) in [(2, 3, 32, 2), (3, 2, 40, 1)]:
        w = (rng.standard_normal((n, k)) * 0.03).astype(np.float32)
        x = bf16_bits(rng.standard_normal((m, k), dtype=np.float32) * 1.7)
        a, b = lora_bf16(r, k, n, 7 * m + n)
        codes, s = fp8.quantize(w)
        y = fp8.w8a8_lora_linear_f64(x, codes, s, a, b, 1.5)
        ex = np.array([[float(v) for v in row] for row in fp8.w8a8_lora_linear_exact(x, codes, s, a, b, 1.5)])
        assert np.allclose(y, ex, rtol=1e-13, atol=0)
        assert np.array_equal(bf16_round(y), bf16_round(ex))
        # quantising activations changes the answer here: W8A8 is not W8A16 in disguise
        assert not np.array_equal(bf16_round(y), fp8.lora_linear(x, codes, s, a, b, 1.5))


def test_w8a8_activation_codes_are_the_weight_encoder_per_token():
    """Token rows quantise exactly like weight rows: torch's float8 cast of fp32(x / s_x)."""
    rng = np.random.default_rng(12)
    x = bf16_bits(rng.standard_normal((9, 200), dtype=np.float32) * 10.0 ** rng.integers(-3, 3, (9, 1)))
    x[4] = 0
    x8, sx = fp8.quantize_activations(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(sx, (np.max(np.abs(xf), axis=1) / np.float32(448)).astype(np.float32))
    q = np.where(sx[:, None] > 0, xf / np.where(sx > 0, sx, 1)[:, None], 0).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(x8, np.where((ref & 0x7F) == 0, 0, ref))
    assert not x8[4].any() and sx[4] == 0


def test_w8a8_equals_w8a16_on_grid_tokens():
    """Tokens already on a scaled E4M3 grid quantise losslessly, so W8A8 = W8A16 exactly.

    The shifts make s_x = 2^-j differ from 1 per row: a dropped or misplaced
    activation scale (or a transposed scale vector) breaks the equality.
    """
    rng = np.random.default_rng(13)
    m, n, k, r = 5, 7, 96, 3
    x = _grid_rows(rng, m, k, [3, 7, 0, 12, 5])
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    a, b = lora_bf16(r, k, n, 99)
    codes, s = fp8.quantize(w)
    x8, sx = fp8.quantize_activations(x)
    assert np.array_equal(sx, np.float32(2.0) ** -np.array([3, 7, 0, 12, 5], np.float32))
    want = fp8.lora_linear_f64(x, codes, s, a, b, 2.0)
    assert np.array_equal(fp8.w8a8_lora_linear_f64(x, codes, s, a, b, 2.0), want)
    # the same check catches a planted slip: the activation scale left out
    wrong = fp8.dequantize(x8, np.ones_like(sx)) @ fp8.dequantize(codes, s).T
    assert not np.allclose(wrong, fp8.lora_linear_f64(x, codes, s), rtol=1e-3)


def test_w8a8_error_bound_against_w8a16():
    """|W8A8 - W8A16| <= sum_k |x - deq(x8)| |deq(w8)| <= sum_k half-step * s_x * |deq(w8)|."""
    rng = np.random.default_rng(14)
    m, n, k = 6, 11, 256
    x = bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    codes, s = fp8.quantize(w)
    x8, sx = fp8.quantize_activations(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q = np.abs(xf) / sx[:, None].astype(np.float64)
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    half = 0.5 * 2.0 ** (e - 3) * sx[:, None]
    dx = np.abs(xf - fp8.dequantize(x8, sx))
    assert np.all(dx <= half * (1 + 1e-6))
    bound = (dx @ np.abs(fp8.dequantize(codes, s)).T)
    diff = np.abs(fp8.w8a8_lora_linear_f64(x, codes, s) - fp8.lora_linear_f64(x, codes, s))
    assert np.all(diff <= bound * (1 + 1e-9) + 1e-300)
    assert np.any(diff > 0)


def test_w8a8_magnitudes_bound_the_product():
    rng = np.random.default_rng(15)
    x = bf16_bits(rng.standard_normal((4, 64), dtype=np.float32))
    w = (rng.standard_normal((5, 64)) * 0.02).astype(np.float32)
    a, b = lora_bf16(2, 64, 5, 3)
    codes, s = fp8.quantize(w)
    base, lora = fp8.w8a8_magnitude_f64(x, codes, s, a, b, -2.0)
    y = fp8.w8a8_lora_linear_f64(x, codes, s, a, b, -2.0)
    assert np.all(np.abs(y) <= (base + lora) * (1 + 1e-12))
    assert np.all(base > 0) and np.all(lora > 0)
    y0 = fp8.w8a8_lora_linear_f64(x, codes, s)
    assert np.all(np.abs(y0) <= base * (1 + 1e-12))
