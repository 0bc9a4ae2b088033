"""GPU parity of the AQN RMSNorm folded into one NVFP4 + LoRA linear (the qkv fold) vs the oracle: the norm
oracle's bf16 tokens fed to the linear oracle."""
import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr
from oracle import aqn, linear, nvfp4
from oracle.numerics import bf16_bits_of, bf16_round, bf16_to_f64, rel_l2
from workloads import LORA_SCALE, QWEN25_7B, activations_bf16, lora_bf16, normal_f32, tensor_seed

from gpu_util import (REL_L2_TOL, accumulation_slack, assert_elementwise, assert_guards, bf16_from_dev, bf16_to_dev,
                      bf16_ulp, device, guarded, nvfp4_to_dev, say)

pytestmark = pytest.mark.gpu

SIGMA, SEED, STEP, NORM_ID, EPS = 1e-2, 3, 1, 4, 1e-6


def _norm_case(m, k, seed):
    x = activations_bf16(m, k, seed)
    w = (1.0 + 0.1 * np.random.default_rng(seed).standard_normal(k)).astype(np.float32)
    return x, w


def _run(dev, x, w, q, a, b, s):
    wq = nvfp4_to_dev(*q, dev)
    at = bf16_to_dev(a, dev) if a is not None else None
    bt = bf16_to_dev(b, dev) if b is not None else None
    buf, y = guarded((x.shape[0], wq.n), torch.bfloat16, dev)
    fr.aqn_lora_linear(bf16_to_dev(x, dev), torch.from_numpy(w).to(dev), SIGMA, SEED, STEP, NORM_ID, EPS, wq, at, bt,
                       s, out=y)
    torch.cuda.synchronize()
    assert_guards(buf, "folded linear output")
    return bf16_from_dev(y)


def _flip_slack(v, q, a, b, s, rows=None):
    """Bound on what normalised tokens rounded the other way can change. The device forms x r_m w in fp32 (r_m
    from its own fp32 sum of squares), the oracle in float64: where the exact value v lies within 2^-18 of its
    magnitude from a bf16 rounding midpoint, the two may round to neighbouring bf16 values (one ulp apart).
    Each such token element moves an output by at most one ulp times |W| plus |s| |B| |A| along its k."""
    ulp = bf16_ulp(v)
    frac = np.abs(v) / ulp
    frac -= np.floor(frac)
    amb = np.abs(frac - 0.5) * ulp <= 2.0 ** -18 * np.abs(v)
    codes, scales, s_t = q
    if rows is not None:
        codes, scales = np.asarray(codes)[rows], np.asarray(scales)[rows]
        b = None if b is None else np.asarray(b)[rows]
    c = np.abs(nvfp4.dequantize(codes, scales, s_t))
    if a is not None and np.asarray(a).shape[0]:
        c = c + abs(s) * (np.abs(bf16_to_f64(b)) @ np.abs(bf16_to_f64(a)))
    return np.where(amb, ulp, 0.0) @ c.T


def _check(y_bits, x, w, q, a, b, s, what, rows=None):
    wn = aqn.noisy_weight(w, SIGMA, SEED, STEP, NORM_ID)
    v = aqn.rmsnorm_f64(x, wn, EPS)  # the normalised tokens before their bf16 rounding
    xn = bf16_bits_of(bf16_round(v))
    want = linear.lora_linear(xn, *q, a, b, s, rows=rows)
    got = bf16_to_f64(y_bits)
    err = rel_l2(got, want)
    say(f"  {what}: rel-L2 {err:.3e}")
    assert err <= REL_L2_TOL, f"{what}: rel-L2 {err}"
    base, lora = linear.lora_linear_magnitude_f64(xn, *q, a, b, s, rows=rows)
    terms = x.shape[1] + (0 if a is None else np.asarray(a).shape[0])
    slack = accumulation_slack(base, lora, terms) + _flip_slack(v, q, a, b, s, rows=rows)
    assert_elementwise(got, want, slack, what)


@pytest.mark.parametrize("shape", [(1, 40, 144, 4), (5, 37, 208, 0), (16, 64, 1040, 8), (17, 100, 512, 32),
                                   (40, 131, 4112, 16), (64, 72, 3584, 32), (100, 40, 16384, 8),
                                   (128, 96, 5120, 16)])
def test_folded_linear_ragged(shape):
    """Ragged widths (n % 16 != 0), K tails past a 128-chunk, every token-tile count (1, 2, 4, 8 tiles of 16),
    no adapters, the widest norm (k = 16384) and the 32B hidden size at 128 tokens."""
    m, n, k, r = shape
    dev = device()
    say(f"AQN-folded linear m={m} n={n} k={k} r={r}")
    seed = 11 * m + n + k + r
    x, w = _norm_case(m, k, seed)
    q = nvfp4.quantize(normal_f32((n, k), 0.05, seed + 1))
    a, b = lora_bf16(r, k, n, seed + 2, std=0.02) if r else (None, None)
    y = _run(dev, x, w, q, a, b, LORA_SCALE)
    _check(y, x, w, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r}")


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_folded_qkv_full_size_7b(m):
    """The 7B qkv projection (4608 x 3584, r = 32) at the decode token counts; sampled output features."""
    dev = device()
    n, k = QWEN25_7B["qkv"]
    x, w = _norm_case(m, k, 70 + m)
    q = nvfp4.quantize(normal_f32((n, k), 0.02, tensor_seed(10, 0, "qkv")))
    a, b = lora_bf16(32, k, n, 71 + m, std=0.01)
    say(f"AQN-folded qkv 7B {n}x{k}, m={m}")
    y = _run(dev, x, w, q, a, b, LORA_SCALE)
    rows = np.sort(np.random.default_rng(m).choice(n, 256, replace=False))
    _check(y[:, rows], x, w, q, a, b, LORA_SCALE, f"7B qkv m={m}", rows=rows)


def test_folded_equals_norm_then_linear_up_to_rounding():
    """The fold against the two launches it replaces (fp4rl_aqn_rmsnorm, then fp4rl_fp4_lora_linear), both on
    the device: the same values up to the order of the fp32 sums and the normalised tokens' rounding."""
    dev = device()
    m, n, k, r = 32, 4608, 3584, 32
    x, w = _norm_case(m, k, 90)
    q = nvfp4.quantize(normal_f32((n, k), 0.02, 91))
    a, b = lora_bf16(r, k, n, 92, std=0.01)
    wq = nvfp4_to_dev(*q, dev)
    xt, wt = bf16_to_dev(x, dev), torch.from_numpy(w).to(dev)
    at, bt = bf16_to_dev(a, dev), bf16_to_dev(b, dev)
    folded = fr.aqn_lora_linear(xt, wt, SIGMA, SEED, STEP, NORM_ID, EPS, wq, at, bt, LORA_SCALE)
    xn = fr.aqn_rmsnorm(xt, wt, SIGMA, SEED, STEP, NORM_ID, EPS)
    two = fr.fp4_lora_linear(xn, wq, at, bt, LORA_SCALE)
    torch.cuda.synchronize()
    err = rel_l2(bf16_to_f64(bf16_from_dev(folded)), bf16_to_f64(bf16_from_dev(two)))
    say(f"  folded vs norm + linear: rel-L2 {err:.3e}")
    assert err <= REL_L2_TOL
