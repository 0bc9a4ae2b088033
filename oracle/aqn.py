"""Adaptive Quantization Noise (AQN) RMSNorm — oracle (test infrastructure only).

What it follows: QeRL explainer (lifetechia), section "Adaptive Quantization
Noise (AQN)":

* "How AQN works": an exponential scheduler injects large noise early in
  training and decays it toward small noise late.
* "Zero overhead: integration into layer normalisation" (the equation there):
  the noise vector is folded into the RMSNorm scale, W_noise = Z_noise + w,
  and the norm computes W_noise * x / sqrt(sum(x^2) + delta). Channel-wise
  additive noise on the weight becomes row-wise multiplicative noise on the
  next linear's input.

Readings taken:

* the normaliser is the mean of squares (root-MEAN-square; the printed
  equation lost the 1/d) — ``sum_mode=True`` gives the literal printed form;
* Z_noise ~ N(0, sigma_k^2) is ONE fp vector of length d per norm and stage,
  shared by all tokens, redrawn when the stage k changes;
* sigma_k = sigma_start * (sigma_end / sigma_start)^(k / (K-1)), k = 0..K-1;
* the Gaussian draw is counter-based so both sides can regenerate it:
  Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
  as 1, 2, 3", SC'11) with counter (q, norm_id, step_lo, step_hi) and key
  (seed_lo, seed_hi), then Box-Muller on 24-bit uniforms (this library's own
  convention, stated in ``philox_normal``).

Pins (tests/test_oracle_aqn.py): Philox words against torch's own
Philox4x32-10 engine (ATen/core/PhiloxRNGEngine.h, compiled on the host);
Kolmogorov-Smirnov and moment tests of the normals; sigma = 0 against
torch.nn.functional.rms_norm; the schedule's end points and constant ratio;
hand-worked golden rows (tests/golden/rmsnorm_rows.txt).
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import bf16_round, bf16_to_f64

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def sigma_schedule(sigma_start: float, sigma_end: float, k: int, num_stages: int) -> np.float32:
    """Exponentially decaying noise level of stage k (fp64 formula, fp32 result)."""
    if num_stages < 1 or not (0 <= k < num_stages):
        raise ValueError("need 0 <= k < num_stages")
    if num_stages == 1:
        return np.float32(sigma_start)
    frac = k / (num_stages - 1)
    return np.float32(sigma_start * (sigma_end / sigma_start) ** frac)


def philox4x32_10(counters, key) -> np.ndarray:
    """Philox4x32 with 10 rounds on an array of 4-word counters.

    counters: [n, 4] uint32; key: (k0, k1). One round maps
    (c0, c1, c2, c3) -> (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,
    lo(M0*c0)); the key is bumped by the Weyl constants between rounds.
    """
    c = np.asarray(counters, dtype=np.uint64).reshape(-1, 4).copy()
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for rnd in range(10):
        p0 = m0 * c[:, 0]
        p1 = m1 * c[:, 2]
        n0 = ((p1 >> np.uint64(32)) ^ c[:, 1] ^ k0) & _MASK32
        n1 = p1 & _MASK32
        n2 = ((p0 >> np.uint64(32)) ^ c[:, 3] ^ k1) & _MASK32
        n3 = p0 & _MASK32
        c = np.stack([n0, n1, n2, n3], axis=1)
        k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
        k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
    return c.astype(np.uint32)


def philox_words(seed: int, step: int, norm_id: int, n_blocks: int) -> np.ndarray:
    """Raw Philox output for counter blocks q = 0..n_blocks-1: [n_blocks, 4] uint32."""
    q = np.arange(n_blocks, dtype=np.uint64)
    ctr = np.zeros((n_blocks, 4), dtype=np.uint64)
    ctr[:, 0] = q & _MASK32
    ctr[:, 1] = np.uint64(norm_id & 0xFFFFFFFF)
    ctr[:, 2] = np.uint64(step & 0xFFFFFFFF)
    ctr[:, 3] = np.uint64((step >> 32) & 0xFFFFFFFF)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return philox4x32_10(ctr, key)


def philox_normal(seed: int, step: int, norm_id: int, d: int) -> np.ndarray:
    """Standard normals z[0:d] (float64) from the counter stream.

    Block q gives words (o0, o1, o2, o3); each pair (a, b) in ((o0, o1),
    (o2, o3)) becomes u1 = ((a >> 8) + 1) * 2^-24 in (0, 1] and
    u2 = (b >> 8) * 2^-24 in [0, 1), then Box-Muller:
    rho = sqrt(-2 ln u1), z = rho cos(2 pi u2) and rho sin(2 pi u2).
    z[4q .. 4q+3] = (cos of pair 0, sin of pair 0, cos of pair 1, sin of pair 1).
    """
    nb = (d + 3) // 4
    w = philox_words(seed, step, norm_id, nb).astype(np.float64)
    a = np.floor(w[:, 0::2] / 256.0)       # (a >> 8) for the two pairs
    b = np.floor(w[:, 1::2] / 256.0)
    u1 = (a + 1.0) * 2.0 ** -24
    u2 = b * 2.0 ** -24
    rho = np.sqrt(-2.0 * np.log(u1))
    zc = rho * np.cos(2.0 * math.pi * u2)
    zs = rho * np.sin(2.0 * math.pi * u2)
    z = np.empty((nb, 4), dtype=np.float64)
    z[:, 0] = zc[:, 0]
    z[:, 1] = zs[:, 0]
    z[:, 2] = zc[:, 1]
    z[:, 3] = zs[:, 1]
    return z.ravel()[:d]


def noisy_weight(w, sigma: float, seed: int, step: int, norm_id: int) -> np.ndarray:
    """W_noise = w + sigma * Z_noise, float64 [d]."""
    w = np.asarray(w, dtype=np.float64)
    z = philox_normal(seed, step, norm_id, w.shape[0])
    return w + np.float64(np.float32(sigma)) * z


def rmsnorm_f64(x_bits, w_eff, eps: float, sum_mode: bool = False) -> np.ndarray:
    """Unrounded w_eff * x / sqrt(mean(x^2) + eps) (or sum(x^2) if sum_mode)."""
    x = bf16_to_f64(x_bits)
    d = x.shape[-1]
    ss = np.sum(x * x, axis=-1, keepdims=True)
    ms = ss if sum_mode else ss / d
    return np.asarray(w_eff, dtype=np.float64) * x / np.sqrt(ms + np.float64(np.float32(eps)))


def aqn_rmsnorm(x_bits, w, sigma: float, seed: int, step: int, norm_id: int,
                eps: float, sum_mode: bool = False):
    """bf16-rounded AQN RMSNorm output [M, d] and the noisy weight [d] (float64)."""
    wn = noisy_weight(w, sigma, seed, step, norm_id)
    return bf16_round(rmsnorm_f64(x_bits, wn, eps, sum_mode)), wn
