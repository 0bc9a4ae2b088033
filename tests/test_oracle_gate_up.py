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
