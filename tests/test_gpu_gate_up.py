"""GPU parity of the fused gate/up projections with the SiLU-gated product vs the oracle."""
import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr
from oracle import gate_up as gu, nvfp4
from oracle.numerics import bf16_to_f64, rel_l2
from workloads import LORA_SCALE, QWEN25_7B, activations_bf16, lora_bf16, normal_f32, tensor_seed

from gpu_util import (REL_L2_TOL, accumulation_slack, assert_elementwise, assert_guards, bf16_from_dev, bf16_to_dev,
                      bf16_ulp, device, guarded, nvfp4_to_dev, say)
from oracle import linear

FUSED_MAX_TOKENS = 16  # above: two linears with bf16 outputs, then the gated product

pytestmark = pytest.mark.gpu


def _run(dev, x, g, u, lg, lu, s):
    wg, wu = nvfp4_to_dev(*g, dev), nvfp4_to_dev(*u, dev)
    lgd = tuple(bf16_to_dev(t, dev) for t in lg) if lg is not None else None
    lud = tuple(bf16_to_dev(t, dev) for t in lu) if lu is not None else None
    buf, h = guarded((x.shape[0], g[0].shape[0]), torch.bfloat16, dev)
    fr.fp4_gate_up_silu(bf16_to_dev(x, dev), wg, wu, lgd, lud, s, out=h)
    torch.cuda.synchronize()
    assert_guards(buf, "gate/up output")
    return bf16_to_f64(bf16_from_dev(h))


def _check(got, x, g, u, lg, lu, s, what, rows=None):
    """rel-L2 against the form the token count selects, and every element within 2 bf16 ulps plus the
    propagated accumulation bound of each projection (and, on the two-step path, one bf16 ulp of each of
    g and u, whose rounding may land on the other side of a midpoint)."""
    m = x.shape[0]
    ag, bg = lg or (None, None)
    au, bu = lu or (None, None)
    two = m > FUSED_MAX_TOKENS
    form = gu.gate_up_two_step if two else gu.gate_up
    want = form(x, g, u, ag, bg, au, bu, s, rows=rows)
    err = rel_l2(got, want)
    say(f"  {what} ({'two linears' if two else 'fused'}): rel-L2 {err:.3e}")
    assert err <= REL_L2_TOL
    yg = linear.lora_linear_f64(x, *g, ag, bg, s, rows=rows)
    yu = linear.lora_linear_f64(x, *u, au, bu, s, rows=rows)
    terms = x.shape[1] + (0 if ag is None else ag.shape[0])
    dg = accumulation_slack(*linear.lora_linear_magnitude_f64(x, *g, ag, bg, s, rows=rows), terms)
    du = accumulation_slack(*linear.lora_linear_magnitude_f64(x, *u, au, bu, s, rows=rows), terms)
    if two:
        dg = dg + bf16_ulp(yg)
        du = du + bf16_ulp(yu)
    slack = 1.1 * np.abs(yu) * dg + np.abs(gu.silu(yg)) * du + 1.1 * dg * du
    assert_elementwise(got, want, slack, what)


@pytest.mark.parametrize("shape", [(1, 16, 16, 0), (3, 40, 144, 4), (16, 64, 256, 8), (17, 100, 512, 32),
                                   (33, 72, 1040, 5), (64, 130, 384, 16), (65, 48, 208, 64), (128, 64, 4112, 8),
                                   (100, 37, 272, 3), (40, 4101, 1040, 8)])
def test_ragged_shapes(shape):
    m, n, k, r = shape
    dev = device()
    say(f"gate/up SiLU m={m} n={n} k={k} r={r}")
    seed = m + n + k + r
    x = activations_bf16(m, k, seed)
    g = nvfp4.quantize(normal_f32((n, k), 0.05, seed + 1))
    u = nvfp4.quantize(normal_f32((n, k), 0.05, seed + 2))
    lg = lora_bf16(r, k, n, seed + 3, std=0.02) if r else None
    lu = lora_bf16(r, k, n, seed + 4, std=0.02) if r else None
    got = _run(dev, x, g, u, lg, lu, LORA_SCALE)
    _check(got, x, g, u, lg, lu, LORA_SCALE, f"{m}x{n}x{k} r{r}")


@pytest.mark.parametrize("m", [1, 16, 17, 32, 128])
def test_full_size_7b(m):
    """7B gate and up (18944 x 3584), r = 32, x with outlier channels; sampled output features."""
    dev = device()
    n, k = QWEN25_7B["gate"]
    x = activations_bf16(m, k, 50 + m, outlier_frac=0.001)
    g = nvfp4.quantize(normal_f32((n, k), 0.02, tensor_seed(8, 0, "gate")))
    u = nvfp4.quantize(normal_f32((n, k), 0.02, tensor_seed(8, 0, "up")))
    lg = lora_bf16(32, k, n, 51, std=0.01)
    lu = lora_bf16(32, k, n, 52, std=0.01)
    say(f"gate/up SiLU 7B {n}x{k}, m={m}")
    got = _run(dev, x, g, u, lg, lu, LORA_SCALE)
    rows = np.sort(np.random.default_rng(m).choice(n, 256, replace=False))
    _check(got[:, rows], x, g, u, lg, lu, LORA_SCALE, f"7B m={m}", rows=rows)


def _aqn_case(m, k, seed):
    x = activations_bf16(m, k, seed)
    w = (1.0 + 0.1 * np.random.default_rng(seed).standard_normal(k)).astype(np.float32)
    return x, w


@pytest.mark.parametrize("shape", [(1, 16, 64, 0), (5, 40, 144, 4), (16, 64, 1040, 8), (40, 100, 512, 32),
                                   (128, 64, 256, 5), (3, 37, 208, 4), (70, 131, 4112, 16),
                                   (128, 72, 5120, 16), (100, 40, 16384, 8), (65, 24, 16384, 4)])
def test_aqn_folded_ragged(shape):
    """The AQN RMSNorm folded into gate/up equals the norm oracle feeding the gate/up oracle. The last three
    shapes are the 32B hidden size at 128 tokens and the widest norm (k = 16384: 64 KB of noisy weight in LDS
    beside the 64 KB reduction buffer of the 8-token-tile launch)."""
    from oracle import aqn
    from oracle.numerics import bf16_bits_of

    m, n, k, r = shape
    dev = device()
    say(f"AQN-folded gate/up SiLU m={m} n={n} k={k} r={r}")
    seed = 7 * m + n + k + r
    x, w = _aqn_case(m, k, seed)
    sigma, rseed, step, norm_id, eps = 1e-2, 3, 1, 5, 1e-6
    g = nvfp4.quantize(normal_f32((n, k), 0.05, seed + 1))
    u = nvfp4.quantize(normal_f32((n, k), 0.05, seed + 2))
    lg = lora_bf16(r, k, n, seed + 3, std=0.02) if r else None
    lu = lora_bf16(r, k, n, seed + 4, std=0.02) if r else None
    wg, wu = nvfp4_to_dev(*g, dev), nvfp4_to_dev(*u, dev)
    lgd = tuple(bf16_to_dev(t, dev) for t in lg) if r else None
    lud = tuple(bf16_to_dev(t, dev) for t in lu) if r else None
    h = fr.aqn_gate_up_silu(bf16_to_dev(x, dev), torch.from_numpy(w).to(dev), sigma, rseed, step, norm_id, eps, wg,
                            wu, lgd, lud, LORA_SCALE)
    torch.cuda.synchronize()
    xn, _ = aqn.aqn_rmsnorm(x, w, sigma, rseed, step, norm_id, eps)
    want = gu.gate_up(bf16_bits_of(xn), g, u, *(lg or (None, None)), *(lu or (None, None)), LORA_SCALE)
    err = rel_l2(bf16_to_f64(bf16_from_dev(h)), want)
    say(f"  rel-L2 {err:.3e}")
    assert err <= REL_L2_TOL


@pytest.mark.parametrize("m", [1, 16])
def test_aqn_folded_full_size_7b(m):
    from oracle import aqn
    from oracle.numerics import bf16_bits_of

    dev = device()
    n, k = QWEN25_7B["gate"]
    x, w = _aqn_case(m, k, 60 + m)
    g = nvfp4.quantize(normal_f32((n, k), 0.02, tensor_seed(9, 0, "gate")))
    u = nvfp4.quantize(normal_f32((n, k), 0.02, tensor_seed(9, 0, "up")))
    lg = lora_bf16(32, k, n, 61, std=0.01)
    lu = lora_bf16(32, k, n, 62, std=0.01)
    say(f"AQN-folded gate/up SiLU 7B {n}x{k}, m={m}")
    h = fr.aqn_gate_up_silu(bf16_to_dev(x, dev), torch.from_numpy(w).to(dev), 1e-2, 4, 0, 2, 1e-6,
                            nvfp4_to_dev(*g, dev), nvfp4_to_dev(*u, dev),
                            tuple(bf16_to_dev(t, dev) for t in lg), tuple(bf16_to_dev(t, dev) for t in lu), LORA_SCALE)
    torch.cuda.synchronize()
    xn, _ = aqn.aqn_rmsnorm(x, w, 1e-2, 4, 0, 2, 1e-6)
    rows = np.sort(np.random.default_rng(m).choice(n, 256, replace=False))
    want = gu.gate_up(bf16_bits_of(xn), g, u, *lg, *lu, LORA_SCALE, rows=rows)
    err = rel_l2(bf16_to_f64(bf16_from_dev(h))[:, rows], want)
    say(f"  rel-L2 {err:.3e}")
    assert err <= REL_L2_TOL


def test_workspace_reused_across_the_two_paths():
    """One zero-filled workspace serves fused and two-linear calls in turn, with the same results as fresh ones."""
    dev = device()
    shapes = [(40, 300, 1040, 16), (8, 300, 1040, 16), (128, 300, 4112, 8), (17, 300, 1040, 0), (3, 300, 1040, 16)]
    need = max(fr.fp4_gate_up_silu_workspace_bytes(m, n, k, r) for m, n, k, r in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for (m, n, k, r) in shapes:
        say(f"gate/up shared workspace m={m} n={n} k={k} r={r}")
        seed = 3 * m + k
        x = bf16_to_dev(activations_bf16(m, k, seed), dev)
        wg = nvfp4_to_dev(*nvfp4.quantize(normal_f32((n, k), 0.05, seed + 1)), dev)
        wu = nvfp4_to_dev(*nvfp4.quantize(normal_f32((n, k), 0.05, seed + 2)), dev)
        lg = tuple(bf16_to_dev(v, dev) for v in lora_bf16(r, k, n, seed + 3, std=0.02)) if r else None
        lu = tuple(bf16_to_dev(v, dev) for v in lora_bf16(r, k, n, seed + 4, std=0.02)) if r else None
        h_shared = fr.fp4_gate_up_silu(x, wg, wu, lg, lu, LORA_SCALE, workspace=ws)
        h_fresh = fr.fp4_gate_up_silu(x, wg, wu, lg, lu, LORA_SCALE)
        torch.cuda.synchronize()
        assert torch.equal(h_shared, h_fresh)
