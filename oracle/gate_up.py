"""Fused gate/up projections with the SiLU-gated product — oracle (test infrastructure only).

What it follows: the QeRL explainer's "Zero overhead: folding into layer
normalization" section and the experiments on Qwen2.5 models, whose MLP
block is gated: h = SiLU(gate) * up, with gate and up two linears of the same
input (the pages name the models; the MLP's gating is that architecture's,
not printed on the pages). Each projection is the NVFP4 + LoRA linear of
``oracle.linear`` with its own weights, tensor scale and adapters:

    g = x deq(Wg)^T + s (x Ag^T) Bg^T,   u = x deq(Wu)^T + s (x Au^T) Bu^T
    h = bf16( SiLU(g) * u ),  SiLU(v) = v / (1 + exp(-v))

Reading taken: fused, g and u are not rounded to bf16 before the gate (one
rounding, of h); the oracle evaluates everything in float64.

Two-step form (``gate_up_two_step``): the same product computed from two
separate linear outputs, each already rounded to bf16 as a linear call
returns it, h = bf16(SiLU(bf16(g)) * bf16(u)). It is the definition of the
path that runs the two projections as separate linears (faster from a few
dozen tokens on), and it differs from the fused form only through the two
extra roundings.

Pins (tests/test_oracle_gate_up.py): SiLU closed forms (SiLU(0) = 0,
SiLU(v) - SiLU(-v) = v, SiLU(v) -> v for large v) and torch's CPU
float64 SiLU; composition with the (pinned) forward oracle; zero up weights
and adapters give h = 0; a zero gate gives h = 0 whatever the up. Two-step:
equal to the fused form when g and u are exact in bf16 (power-of-two tensor
scales, one-hot tokens); otherwise within the propagated error of the two
roundings (|SiLU'| <= 1.1).
"""
from __future__ import annotations

import numpy as np

from .linear import lora_linear_f64
from .numerics import bf16_round


def silu(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def gate_up_f64(x_bits, gate, up, a_g=None, b_g=None, a_u=None, b_u=None, lora_scale: float = 0.0,
                rows=None) -> np.ndarray:
    """Unrounded SiLU(g) * u [M, N]; ``gate``/``up`` = (codes, scales, s_t); ``rows`` selects output columns."""
    g = lora_linear_f64(x_bits, *gate, a_g, b_g, lora_scale, rows=rows)
    u = lora_linear_f64(x_bits, *up, a_u, b_u, lora_scale, rows=rows)
    return silu(g) * u


def gate_up(x_bits, gate, up, a_g=None, b_g=None, a_u=None, b_u=None, lora_scale: float = 0.0,
            rows=None) -> np.ndarray:
    """bf16-rounded h (float64 values), the device output's reference."""
    return bf16_round(gate_up_f64(x_bits, gate, up, a_g, b_g, a_u, b_u, lora_scale, rows))


def gate_up_two_step(x_bits, gate, up, a_g=None, b_g=None, a_u=None, b_u=None, lora_scale: float = 0.0,
                     rows=None) -> np.ndarray:
    """bf16(SiLU(bf16(g)) * bf16(u)) (float64 values): the product of two rounded linear outputs."""
    g = bf16_round(lora_linear_f64(x_bits, *gate, a_g, b_g, lora_scale, rows=rows))
    u = bf16_round(lora_linear_f64(x_bits, *up, a_u, b_u, lora_scale, rows=rows))
    return bf16_round(silu(g) * u)
