"""Pins of the fused gate/up + SiLU oracle (CPU only)."""
import numpy as np
import torch

from oracle import gate_up as gu, linear
from oracle.numerics import bf16_round
from oracle.nvfp4 import quantize
from workloads import bf16_bits, lora_bf16, normal_f32


def test_silu_closed_forms_and_torch():
    v = np.linspace(-30, 30, 2001)
    s = gu.silu(v)
    assert gu.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(s - gu.silu(-v), v, rtol=0, atol=1e-12)
    assert np.allclose(gu.silu(np.array([40.0, 60.0])), [40.0, 60.0], rtol=1e-15)
    ref = torch.nn.functional.silu(torch.from_numpy(v)).numpy()
    assert np.allclose(s, ref, rtol=1e-14, atol=1e-300)


def _case(seed, m=4, n=48, k=96, r=4):
    x = bf16_bits(normal_f32((m, k), 1.0, seed))
    g = quantize(normal_f32((n, k), 0.05, seed + 1))
    u = quantize(normal_f32((n, k), 0.05, seed + 2))
    ag, bg = lora_bf16(r, k, n, seed + 3, std=0.05)
    au, bu = lora_bf16(r, k, n, seed + 4, std=0.05)
    return x, g, u, ag, bg, au, bu


def test_composition_with_the_linear_oracle():
    x, g, u, ag, bg, au, bu = _case(1)
    h = gu.gate_up_f64(x, g, u, ag, bg, au, bu, 2.0)
    yg = linear.lora_linear_f64(x, *g, ag, bg, 2.0)
    yu = linear.lora_linear_f64(x, *u, au, bu, 2.0)
    # written out element by element with the closed form of SiLU
    for i in range(4):
        for n in (0, 7, 47):
            want = yg[i, n] / (1.0 + np.exp(-yg[i, n])) * yu[i, n]
            assert np.isclose(h[i, n], want, rtol=1e-14)
    rows = np.array([3, 0, 40])
    assert np.array_equal(gu.gate_up(x, g, u, ag, bg, au, bu, 2.0, rows=rows), bf16_round(h)[:, rows])


def test_zero_cases():
    x, g, u, ag, bg, au, bu = _case(2)
    z = (np.zeros_like(u[0]), np.zeros_like(u[1]), np.float32(0))
    assert not gu.gate_up(x, g, z, ag, bg, au, np.zeros_like(bu), 2.0).any()
    assert not gu.gate_up(x, z, u, ag, np.zeros_like(bg), au, bu, 2.0).any()


def _exact_case(seed, m=6, n=40, k=64):
    """Linear outputs exact in bf16: one-hot power-of-two tokens, tensor scales 2^-7 and 2^-9.

    A product e2m1 * e4m3 block scale * 2^a needs at most 6 significant bits.
    """
    rng = np.random.default_rng(seed)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), rng.integers(0, k, m)] = 2.0 ** rng.integers(-3, 4, m)
    xb = bf16_bits(x)
    def weight(s_t):
        codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
        scales = rng.integers(0x28, 0x50, (n, k // 16), dtype=np.uint8)  # E4M3 2^-2 .. 2^2 range, 4 significant bits
        return codes, scales, np.float32(s_t)
    return xb, weight(2.0 ** -7), weight(2.0 ** -9)


def test_two_step_equals_fused_when_outputs_are_exact():
    x, g, u = _exact_case(5)
    yg = linear.lora_linear_f64(x, *g)
    assert np.array_equal(bf16_round(yg), yg), "the constructed gate outputs are bf16-exact"
    assert np.array_equal(gu.gate_up_two_step(x, g, u), gu.gate_up(x, g, u))


def test_two_step_within_the_rounding_bound():
    """|h2 - SiLU(g) u| <= 1.1 |u| |g - bf16(g)| + |SiLU(g)| |u - bf16(u)| + (2nd order) + half an ulp of h2."""
    x, g, u, ag, bg, au, bu = _case(6, m=8, n=64, k=160, r=8)
    yg = linear.lora_linear_f64(x, *g, ag, bg, 2.0)
    yu = linear.lora_linear_f64(x, *u, au, bu, 2.0)
    exact = gu.silu(yg) * yu
    h2 = gu.gate_up_two_step(x, g, u, ag, bg, au, bu, 2.0)
    dg, du = np.abs(yg - bf16_round(yg)), np.abs(yu - bf16_round(yu))
    half_ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(h2), 1e-300))).astype(int) - 8)
    bound = 1.1 * np.abs(yu) * dg + np.abs(gu.silu(yg)) * du + 1.1 * dg * du + half_ulp
    assert np.all(np.abs(h2 - exact) <= bound * (1 + 1e-9))
    # and the roundings matter: the two forms differ somewhere on this data
    assert not np.array_equal(h2, gu.gate_up(x, g, u, ag, bg, au, bu, 2.0))
    # a planted slip, the gate and up outputs swapped, is far outside the bound
    swapped = bf16_round(gu.silu(bf16_round(yu)) * bf16_round(yg))
    assert np.any(np.abs(swapped - exact) > bound)
