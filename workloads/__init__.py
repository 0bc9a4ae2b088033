"""Seeded synthetic inputs for the NVFP4 + LoRA + AQN hot path.

This module only draws random tensors of the right shapes and distributions.
It holds none of the method's arithmetic (no quantisation, no norm, no
product), so both the CPU oracle and the HIP path can take their inputs from
it without sharing any of the computation under test.

Shapes follow the Qwen2.5 family the QeRL pages train (page 1 "benchmarks and
models": 3B/7B/14B/32B). The datasets the pages evaluate on (GSM8K, MATH 500,
BigMath) are not needed: only shapes and value distributions matter for a
linear layer or a norm, so seeded Gaussian / Student-t tensors stand in.

bf16 tensors are returned as ``numpy.uint16`` bit patterns (round to nearest
even from float32, done by torch's CPU cast).
"""
from __future__ import annotations

import numpy as np

# Per-layer linear shapes (N out-features, K in-features).
QWEN25_7B = {
    "qkv": (4608, 3584),
    "o": (3584, 3584),
    "gate": (18944, 3584),
    "up": (18944, 3584),
    "down": (3584, 18944),
}
QWEN25_14B = {
    "qkv": (7168, 5120),
    "o": (5120, 5120),
    "gate": (13824, 5120),
    "up": (13824, 5120),
    "down": (5120, 13824),
}
QWEN25_32B = {
    "qkv": (7168, 5120),
    "o": (5120, 5120),
    "gate": (27648, 5120),
    "up": (27648, 5120),
    "down": (5120, 27648),
}
MATRIX_INDEX = {"qkv": 0, "o": 1, "gate": 2, "up": 3, "down": 4, "norm1": 5, "norm2": 6}

LORA_SCALE = 2.0        # s in y = x deq(W)^T + s (x A^T) B^T
LORA_STD = 0.01
WEIGHT_STD = 0.02


def tensor_seed(config: int, layer: int, name: str) -> int:
    """Per-tensor seed: config*1_000_003 + 101*layer + matrix index."""
    return config * 1_000_003 + 101 * layer + MATRIX_INDEX[name]


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), RNE, via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal_f32(shape, std: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations_bf16(m: int, k: int, seed: int, outlier_frac: float = 0.0,
                     outlier_gain: float = 20.0) -> np.ndarray:
    """x ~ N(0,1) in bf16; round(outlier_frac*K) whole channels scaled by the gain.

    The outlier channels are drawn once per tensor by a seeded permutation and
    hold for every token (rollout prefill activations with channel outliers).
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    n_out = int(round(outlier_frac * k))
    if n_out:
        ch = rng.permutation(k)[:n_out]
        x[:, ch] *= np.float32(outlier_gain)
    return bf16_bits(x)


def lora_bf16(r: int, k: int, n: int, seed: int, std: float = LORA_STD):
    """LoRA adapters A [r,K], B [N,r] ~ N(0, std) in bf16."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((r, k), dtype=np.float32) * np.float32(std)
    b = rng.standard_normal((n, r), dtype=np.float32) * np.float32(std)
    return bf16_bits(a), bf16_bits(b)


def student_t3_weights_torch(shape, seed: int, device, scale: float = 0.02,
                             outlier_p: float = 1e-4, outlier_gain: float = 50.0):
    """The same heavy-tailed recipe drawn on a device with torch's generator (for timing runs):
    0.02 * z0 / sqrt((z1^2 + z2^2 + z3^2) / 3), Bernoulli(1e-4) positions x50. fp32."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z0 = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    den = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(3):
        den.add_(torch.randn(shape, generator=g, device=device, dtype=torch.float32).square_())
    w = z0.div_(den.div_(3.0).sqrt_()).mul_(scale)
    del den
    hit = torch.rand(shape, generator=g, device=device) < outlier_p
    w[hit] *= outlier_gain
    return w


def student_t3_weights(shape, seed: int, scale: float = 0.02,
                       outlier_p: float = 1e-4, outlier_gain: float = 50.0) -> np.ndarray:
    """Heavy-tailed weights: 0.02 * t(nu=3), Bernoulli(1e-4) positions x50.

    t3 = z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) with i.i.d. standard normals.
    """
    rng = np.random.default_rng(seed)
    z0 = rng.standard_normal(shape, dtype=np.float32)
    chi = np.zeros(shape, dtype=np.float32)
    for _ in range(3):
        z = rng.standard_normal(shape, dtype=np.float32)
        chi += z * z
    w = (z0 / np.sqrt(chi / np.float32(3.0))) * np.float32(scale)
    mask = rng.random(shape, dtype=np.float32) < np.float32(outlier_p)
    w[mask] *= np.float32(outlier_gain)
    return w.astype(np.float32)


def single_linear_config(seed: int = 0):
    """The 256x512 single-linear case, drawn from default_rng(seed) in the order W, x, A, B.

    W fp32 ~N(0,0.02) [256,512]; x bf16 ~N(0,1) [4,512]; A bf16 ~N(0,0.01) [8,512];
    B bf16 ~N(0,0.01) [256,8]; LoRA scale 2.0; AQN RMSNorm over the 512-wide
    input with w = 1, sigma = 1e-2, delta = 1e-6, Philox seed = seed.
    """
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((256, 512), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    x = rng.standard_normal((4, 512), dtype=np.float32)
    a = rng.standard_normal((8, 512), dtype=np.float32) * np.float32(0.01)
    b = rng.standard_normal((256, 8), dtype=np.float32) * np.float32(0.01)
    return {
        "w": w,
        "x": bf16_bits(x),
        "lora_a": bf16_bits(a),
        "lora_b": bf16_bits(b),
        "lora_scale": 2.0,
        "norm_w": np.ones(512, dtype=np.float32),
        "sigma": 1e-2,
        "eps": 1e-6,
        "seed": seed,
        "step": 0,
        "norm_id": 0,
    }


def aqn_sigma_stages(sigma_start: float = 1e-2, sigma_end: float = 5e-4, stages: int = 10):
    """Parameters of the exponential AQN decay used by the 14B stress case."""
    return sigma_start, sigma_end, stages


# --------------------------------------------------------------------------
# Device-side generators (torch), for the large benchmark workloads. These are
# plumbing: they only fill HBM with seeded random numbers.
# --------------------------------------------------------------------------

def torch_normal(shape, std: float, seed: int, device, dtype=None):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    if dtype is not None:
        t = t.to(dtype)
    return t
