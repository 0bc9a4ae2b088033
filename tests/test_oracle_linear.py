"""Pins of the oracle's fused LoRA linear (CPU only)."""
import numpy as np
import torch

from oracle import linear
from oracle.numerics import bf16_round
from oracle.nvfp4 import quantize
from workloads import bf16_bits, lora_bf16


def _case(seed, m, n, k, r, wscale=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * wscale).astype(np.float32)
    x = bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    a, b = lora_bf16(r, k, n, seed + 1)
    return w, x, a, b


def test_float64_path_matches_exact_rationals():
    for seed, (m, n, k, r) in enumerate([(2, 3, 32, 2), (1, 4, 16, 1), (3, 2, 48, 3)]):
        w, x, a, b = _case(seed, m, n, k, r)
        codes, scales, st = quantize(w)
        y64 = linear.lora_linear_f64(x, codes, scales, st, a, b, 2.0)
        exact = linear.lora_linear_exact(x, codes, scales, st, a, b, 2.0)
        ex = np.array([[float(v) for v in row] for row in exact])
        assert np.allclose(y64, ex, rtol=1e-13, atol=0)
        assert np.array_equal(bf16_round(y64), bf16_round(ex))


def test_lora_terms_reduce():
    w, x, a, b = _case(20, 4, 64, 128, 8)
    codes, scales, st = quantize(w)
    base = linear.lora_linear(x, codes, scales, st)
    assert np.array_equal(linear.lora_linear(x, codes, scales, st, a, np.zeros_like(b), 2.0), base)
    assert np.array_equal(linear.lora_linear(x, codes, scales, st, a, b, 0.0), base)
    # W = 0: y is the LoRA product alone; check against torch's CPU float64 matmul
    zc = np.zeros_like(codes)
    zs = np.zeros_like(scales)
    y = linear.lora_linear(x, zc, zs, np.float32(0.0), a, b, 2.0)
    xt = torch.from_numpy((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    at = torch.from_numpy((a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    bt = torch.from_numpy((b.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    ref = 2.0 * torch.matmul(torch.matmul(xt, at.T), bt.T)
    assert np.array_equal(y, bf16_round(ref.numpy()))


def test_homogeneity_and_row_selection():
    w, x, a, b = _case(21, 3, 40, 64, 4)
    codes, scales, st = quantize(w)
    y = linear.lora_linear(x, codes, scales, st, a, b, 2.0)
    x2 = bf16_bits(((x.astype(np.uint32) << 16).view(np.float32) * 2).astype(np.float32))
    y2 = linear.lora_linear(x2, codes, scales, st, a, b, 2.0)
    assert np.array_equal(y2, 2 * y)
    rows = np.array([0, 7, 39, 12])
    assert np.array_equal(linear.lora_linear(x, codes, scales, st, a, b, 2.0, rows=rows), y[:, rows])


def test_base_product_against_torch_dequant():
    # an independent dequantisation: torch CPU float8 decode of the scale bytes
    w, x, _, _ = _case(22, 5, 32, 64, 1)
    codes, scales, st = quantize(w)
    grid = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float64)
    c = torch.from_numpy(codes.astype(np.int64))
    c4 = torch.stack([c & 15, c >> 4], dim=-1).reshape(32, 64)
    val = grid[c4 & 7] * torch.where((c4 & 8) > 0, -1.0, 1.0)
    sb = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64)
    wd = val * sb.repeat_interleave(16, dim=1) * float(st)
    xt = torch.from_numpy((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    ref = bf16_round((xt @ wd.T).numpy())
    assert np.array_equal(linear.lora_linear(x, codes, scales, st), ref)


def test_lora_down_matches_exact_rationals():
    """t = s x A^T term by term in Fractions, on adapters that are not square (r != K)."""
    for seed, (m, k, r, s) in enumerate([(2, 32, 3, 2.0), (3, 16, 5, 0.5), (1, 48, 2, 2.0)]):
        rng = np.random.default_rng(100 + seed)
        x = bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
        a = bf16_bits(rng.standard_normal((r, k), dtype=np.float32) * np.float32(0.05))
        t = linear.lora_down(x, a, s)
        assert t.shape == (m, r)
        ex = np.array([[float(v) for v in row] for row in linear.lora_down_exact(x, a, s)])
        assert np.allclose(t, ex, rtol=1e-13, atol=0)


def test_lora_down_catches_a_dropped_scale_or_transposed_adapter():
    """The pin above would fail for the two plausible slips: s left out, or A used untransposed
    (a square A with A != A^T, so the shapes cannot catch it)."""
    rng = np.random.default_rng(7)
    m, k, s = 3, 16, 2.0
    x = bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    a = bf16_bits(rng.standard_normal((k, k), dtype=np.float32) * np.float32(0.05))
    ex = np.array([[float(v) for v in row] for row in linear.lora_down_exact(x, a, s)])
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    av = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.allclose(linear.lora_down(x, a, s), ex, rtol=1e-13, atol=0)
    assert not np.allclose(xv @ av.T, ex, rtol=1e-6)        # s dropped
    assert not np.allclose(s * (xv @ av), ex, rtol=1e-6)    # A not transposed
    # and t is the LoRA term of the fused linear: zero base weight, B = I_r gives y = bf16(t)
    zc = np.zeros((k, k // 2), np.uint8)
    zs = np.zeros((k, k // 16), np.uint8)
    eye = bf16_bits(np.eye(k, dtype=np.float32))
    y = linear.lora_linear(x, zc, zs, np.float32(0.0), a, eye, s)
    assert np.array_equal(y, bf16_round(ex))


def test_magnitude_sums():
    """On non-negative operands the magnitude sums are the linear itself; elsewhere they bound |y|."""
    rng = np.random.default_rng(9)
    m, n, k, r = 3, 20, 64, 4
    w = np.abs(rng.standard_normal((n, k)).astype(np.float32)) * np.float32(0.02)
    x = bf16_bits(np.abs(rng.standard_normal((m, k), dtype=np.float32)))
    a = bf16_bits(np.abs(rng.standard_normal((r, k), dtype=np.float32)) * np.float32(0.05))
    b = bf16_bits(np.abs(rng.standard_normal((n, r), dtype=np.float32)) * np.float32(0.05))
    codes, scales, st = quantize(w)
    base, lora = linear.lora_linear_magnitude_f64(x, codes, scales, st, a, b, 2.0)
    assert np.allclose(base + lora, linear.lora_linear_f64(x, codes, scales, st, a, b, 2.0), rtol=1e-13)
    assert np.allclose(base, linear.lora_linear_f64(x, codes, scales, st), rtol=1e-13)
    w2, x2, a2, b2 = _case(10, m, n, k, r)
    q2 = quantize(w2)
    base2, lora2 = linear.lora_linear_magnitude_f64(x2, *q2, a2, b2, -2.0)
    y2 = linear.lora_linear_f64(x2, *q2, a2, b2, -2.0)
    assert np.all(np.abs(y2) <= (base2 + lora2) * (1 + 1e-12))
    rows = np.array([3, 0, 19])
    assert np.array_equal(linear.lora_linear_magnitude_f64(x2, *q2, a2, b2, 2.0, rows=rows)[0], base2[:, rows])
