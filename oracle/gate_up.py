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

Pins (tests/test_oracle_gate_up.py): SiLU closed forms (SiLU(0) = 0,
SiLU(v) - SiLU(-v) = v, SiLU(v) -> v for large v) and torch's CPU
float64 SiLU; composition with the (pinned) forward oracle; zero up weights
and adapters give h = 0; a zero gate gives h = 0 whatever the up.
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
