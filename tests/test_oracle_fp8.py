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
