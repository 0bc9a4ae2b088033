"""GPU parity of the LoRA backward through the frozen NVFP4 base (dX, dA, dB) vs the oracle."""
import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr
from oracle import lora_backward as lb, nvfp4
from oracle.numerics import bf16_round, bf16_to_f64, rel_l2
from workloads import LORA_SCALE, QWEN25_7B, activations_bf16, bf16_bits, lora_bf16, normal_f32, tensor_seed

from gpu_util import (REL_L2_TOL, accumulation_slack, assert_elementwise, assert_guards, bf16_from_dev, bf16_to_dev,
                      device, f32_ulp, guarded, nvfp4_to_dev, say)

pytestmark = pytest.mark.gpu

# dA and dB are fp32 sums of exact bf16 products (t and h in fp32): far inside
# the bf16 output tolerance
GRAD_TOL = 1e-5


def _case(m, n, k, r, seed):
    w = normal_f32((n, k), 0.02, seed)
    x = activations_bf16(m, k, seed + 1)
    dy = bf16_bits(normal_f32((m, n), 0.05, seed + 2))
    a, b = lora_bf16(r, k, n, seed + 3, std=0.02)
    return w, x, dy, a, b


def _upload(dev, x, dy, q, a, b):
    xt, dyt, wq = bf16_to_dev(x, dev), bf16_to_dev(dy, dev), nvfp4_to_dev(*q, dev)
    at = bf16_to_dev(a, dev) if a is not None and a.shape[0] else None
    bt = bf16_to_dev(b, dev) if b is not None and b.shape[1] else None
    return xt, dyt, wq, at, bt


def _err(got, want, what, tol):
    err = rel_l2(got, want)
    say(f"  {what}: rel-L2 {err:.3e}")
    assert err <= tol, f"{what}: rel-L2 {err}"


# (m, n, k, r): tokens ragged against the 128-row tiles, features against the
# 64-wide chunks and 128-wide tiles, ranks not a multiple of 8, r = 0
RAGGED = [
    (1, 8, 16, 1), (5, 40, 80, 4), (16, 64, 128, 8), (37, 136, 272, 5), (128, 128, 128, 16),
    (130, 200, 400, 24), (257, 96, 1040, 64), (64, 520, 64, 3), (200, 64, 256, 0), (33, 48, 4112, 256),
]


@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_shapes(shape):
    m, n, k, r = shape
    dev = device()
    say(f"lora backward m={m} n={n} k={k} r={r}")
    w, x, dy, a, b = _case(m, n, k, r, seed=m * 7 + n + k + r)
    q = nvfp4.quantize(w)
    xt, dyt, wq, at, bt = _upload(dev, x, dy, q, a, b)
    bufs = [guarded((m, k), torch.bfloat16, dev), guarded((r, k), torch.float32, dev),
            guarded((n, r), torch.float32, dev)]
    dx, ga, gb = fr.fp4_lora_linear_backward(dyt, xt, wq, at, bt, LORA_SCALE,
                                             out=(bufs[0][1], bufs[1][1] if r else None, bufs[2][1] if r else None))
    torch.cuda.synchronize()
    for (buf, _), what in zip(bufs, ("dX", "dA", "dB")):
        assert_guards(buf, f"backward {what}")
    dx_ref, da_ref, db_ref = lb.lora_linear_backward(dy, x, *q, a if r else None, b if r else None, LORA_SCALE)
    dxb, dxl, da_m, db_m = lb.backward_magnitudes_f64(dy, x, *q, a if r else None, b if r else None, LORA_SCALE)
    dx_got = bf16_to_f64(bf16_from_dev(dx))
    _err(dx_got, dx_ref, "dX", REL_L2_TOL)
    assert_elementwise(dx_got, dx_ref, accumulation_slack(dxb, 0.0 if dxl is None else dxl, n + r), "dX")
    if r:
        da_got, db_got = ga.cpu().numpy().astype(np.float64), gb.cpu().numpy().astype(np.float64)
        _err(da_got, da_ref, "dA", GRAD_TOL)
        _err(db_got, db_ref, "dB", GRAD_TOL)
        # fp32 outputs: their own rounding (2^-24 relative) plus the accumulation over tokens and the
        # rank-space operands' bf16 hi + lo split (2^-15 of the magnitude)
        assert_elementwise(da_got, da_ref, (m + n + 64) * 2.0 ** -24 * da_m + 2.0 ** -15 * da_m, "dA", ulp=f32_ulp)
        assert_elementwise(db_got, db_ref, (m + k + 64) * 2.0 ** -24 * db_m + 2.0 ** -15 * db_m, "dB", ulp=f32_ulp)
    else:
        assert ga is None and gb is None


def test_adapter_gradients_only_and_repeat():
    """dx = NULL computes the same adapter gradients; a second call with the same inputs is bitwise equal."""
    dev = device()
    m, n, k, r = 96, 136, 528, 16
    w, x, dy, a, b = _case(m, n, k, r, seed=11)
    q = nvfp4.quantize(w)
    xt, dyt, wq, at, bt = _upload(dev, x, dy, q, a, b)
    say("lora backward adapters only, and repeat")
    dx1, ga1, gb1 = fr.fp4_lora_linear_backward(dyt, xt, wq, at, bt, LORA_SCALE)
    none, ga2, gb2 = fr.fp4_lora_linear_backward(dyt, xt, wq, at, bt, LORA_SCALE, want_dx=False)
    dx3, ga3, gb3 = fr.fp4_lora_linear_backward(dyt, xt, wq, at, bt, LORA_SCALE)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(ga1, ga2) and torch.equal(gb1, gb2)
    assert torch.equal(dx1, dx3) and torch.equal(ga1, ga3) and torch.equal(gb1, gb3)


def test_empty_sums_write_zeros():
    dev = device()
    k, r = 64, 4
    a, b = lora_bf16(r, k, 16, 3)
    x0 = torch.empty((0, k), dtype=torch.bfloat16, device=dev)
    dy0 = torch.empty((0, 16), dtype=torch.bfloat16, device=dev)
    q = nvfp4.quantize(normal_f32((16, k), 0.02, 4))
    wq = nvfp4_to_dev(*q, dev)
    say("lora backward m = 0")
    dx, ga, gb = fr.fp4_lora_linear_backward(dy0, x0, wq, bf16_to_dev(a, dev), bf16_to_dev(b, dev), 2.0)
    torch.cuda.synchronize()
    assert dx.shape == (0, k) and not ga.any() and not gb.any()


def _full_size(name, m, r, seed):
    """Full 7B shapes: every dA row and sampled dX columns and dB rows, each against the oracle."""
    dev = device()
    n, k = QWEN25_7B[name]
    w = normal_f32((n, k), 0.02, tensor_seed(seed, 0, name))
    x = activations_bf16(m, k, seed + 1)
    dy = bf16_bits(normal_f32((m, n), 0.05, seed + 2))
    a, b = lora_bf16(r, k, n, seed + 3, std=0.02)
    q = nvfp4.quantize(w)
    say(f"lora backward 7B {name} {n}x{k}, m={m}, r={r}")
    xt, dyt, wq, at, bt = _upload(dev, x, dy, q, a, b)
    dx, ga, gb = fr.fp4_lora_linear_backward(dyt, xt, wq, at, bt, LORA_SCALE)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    cols = np.sort(rng.choice(k, 96, replace=False))
    rows = np.sort(rng.choice(n, 128, replace=False))
    h, da_ref, db_ref = lb.adapter_terms_f64(dy, x, a, b, LORA_SCALE, b_rows=rows)
    want = bf16_round(lb.dx_columns_f64(dy, *q, cols, a, h))  # the oracle's dX is rounded once to bf16
    got = bf16_to_f64(bf16_from_dev(dx)[:, cols])
    _err(got, want, f"{name} dX ({len(cols)} columns)", REL_L2_TOL)
    _err(ga.cpu().numpy().astype(np.float64), da_ref, f"{name} dA", GRAD_TOL)
    _err(gb.cpu().numpy()[rows].astype(np.float64), db_ref, f"{name} dB ({len(rows)} rows)", GRAD_TOL)


def test_full_size_7b_gate():
    _full_size("gate", 1024, 64, 40)


def test_full_size_7b_down():
    _full_size("down", 512, 32, 41)


def test_full_size_7b_gate_8192_tokens():
    """The configuration the bench times: 7B gate, M = 8192, r = 32 (sampled dX columns, all of dA,
    sampled dB rows)."""
    _full_size("gate", 8192, 32, 42)
