"""GPU parity of the FP8 (E4M3, per-row scale) quantiser and W8A16 LoRA linear vs the oracle."""
import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr
from oracle import fp8
from oracle.numerics import bf16_round, bf16_to_f64, rel_l2
from workloads import (LORA_SCALE, QWEN25_7B, activations_bf16, bf16_bits, bf16_values, lora_bf16, normal_f32,
                       tensor_seed)

from gpu_util import (REL_L2_TOL, accumulation_slack, assert_elementwise, assert_guards, bf16_from_dev, bf16_to_dev,
                      device, f32_to_dev, guarded, say, u8_to_dev)

pytestmark = pytest.mark.gpu


def _quantize_dev(w, dev, bf16=False):
    wt = bf16_to_dev(bf16_bits(w), dev) if bf16 else f32_to_dev(w, dev)
    q = fr.fp8_quantize(wt)
    torch.cuda.synchronize()
    return q.codes.cpu().numpy(), q.scales.cpu().numpy()


def _assert_exact(got, want, what):
    (c, s), (c0, s0) = got, want
    assert np.array_equal(s.view(np.uint32), s0.view(np.uint32)), f"{what}: row scales differ"
    nbad = int(np.count_nonzero(c != c0))
    assert nbad == 0, f"{what}: {nbad} code bytes differ"


@pytest.mark.parametrize("shape", [(1, 16), (37, 80), (130, 272), (256, 4096), (3, 5136)])
def test_quantize_ragged(shape):
    dev = device()
    w = normal_f32(shape, 0.02, shape[0] + shape[1])
    say(f"fp8 quantize {shape}")
    _assert_exact(_quantize_dev(w, dev), fp8.quantize(w), str(shape))
    _assert_exact(_quantize_dev(w, dev, bf16=True), fp8.quantize(bf16_values(bf16_bits(w))), f"{shape} bf16")


def test_quantize_edge_values():
    dev = device()
    rng = np.random.default_rng(8)
    cases = {
        "zero_rows": np.zeros((4, 64), np.float32),
        "tiny": (rng.standard_normal((8, 64)) * 1e-38).astype(np.float32),
        "huge": (rng.standard_normal((8, 64)) * 1e37).astype(np.float32),
        "wide_range": (rng.standard_normal((16, 128)) * 10.0 ** rng.integers(-12, 12, (16, 128))).astype(np.float32),
        "outlier": np.where(np.arange(32 * 96).reshape(32, 96) % 97 == 3, 50.0,
                            rng.standard_normal((32, 96)) * 1e-3).astype(np.float32),
    }
    # every E4M3 magnitude, its midpoints and fp32 neighbours, in rows whose amax is 448 s
    grid = np.array([float(fp8.e4m3_value(b)) for b in range(0x7F)])
    mids = (grid[:-1] + grid[1:]) / 2
    pts = np.concatenate([grid, mids]).astype(np.float32)
    vals = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    vals = vals[: len(vals) // 16 * 16]
    row = np.concatenate([[448.0], vals[1:]]).astype(np.float32)
    cases["grid_and_midpoints"] = np.stack([row, -row, row * np.float32(0.5)])
    for name, w in cases.items():
        say(f"fp8 quantize edge case {name}")
        _assert_exact(_quantize_dev(w, dev), fp8.quantize(w), name)


def _linear_case(m, n, k, r, seed):
    w = normal_f32((n, k), 0.02, seed)
    x = activations_bf16(m, k, seed + 1)
    a, b = lora_bf16(r, k, n, seed + 2, std=0.01)
    return w, x, a, b


@pytest.mark.parametrize("shape", [(1, 8, 16, 0), (3, 40, 80, 4), (17, 100, 512, 32), (64, 520, 1040, 8),
                                   (130, 200, 400, 24), (257, 96, 272, 64), (5, 4100, 32, 1),
                                   # output widths not a multiple of 4: the scalar tails of every path
                                   (5, 37, 80, 4), (40, 4101, 1040, 8), (130, 37, 272, 8), (300, 1027, 2064, 5)])
def test_linear_ragged(shape):
    m, n, k, r = shape
    dev = device()
    say(f"fp8 linear m={m} n={n} k={k} r={r}")
    w, x, a, b = _linear_case(m, n, k, r, seed=m + n + k + r)
    codes, s = fp8.quantize(w)
    w8 = fr.FP8Weight(u8_to_dev(codes, dev), f32_to_dev(s, dev))
    at = bf16_to_dev(a, dev) if r else None
    bt = bf16_to_dev(b, dev) if r else None
    buf, y = guarded((m, n), torch.bfloat16, dev)
    fr.fp8_lora_linear(bf16_to_dev(x, dev), w8, at, bt, LORA_SCALE, out=y)
    torch.cuda.synchronize()
    assert_guards(buf, "fp8 linear output")
    ref = fp8.lora_linear(x, codes, s, a if r else None, b if r else None, LORA_SCALE)
    got = bf16_to_f64(bf16_from_dev(y))
    err = rel_l2(got, ref)
    say(f"  rel-L2 {err:.3e}")
    assert err <= REL_L2_TOL
    # per element: |x| |W| and the LoRA magnitude, both from the oracle's dequantised rows
    xa = np.abs(bf16_to_f64(x))
    base = xa @ np.abs(fp8.dequantize(codes, s)).T
    lora = 0.0
    if r:
        lora = abs(LORA_SCALE) * ((xa @ np.abs(bf16_to_f64(a)).T) @ np.abs(bf16_to_f64(b)).T)
    assert_elementwise(got, ref, accumulation_slack(base, lora, k + r), "fp8 linear")


@pytest.mark.parametrize("m", [1, 32, 1024, 8192])
def test_linear_full_size_7b_gate(m):
    """GPU quantiser feeding the GPU linear at the 7B gate shape; sampled output columns vs the oracle."""
    dev = device()
    n, k = QWEN25_7B["gate"]
    w = normal_f32((n, k), 0.02, tensor_seed(7, 0, "gate"))
    x = activations_bf16(m, k, 9, outlier_frac=0.001)
    a, b = lora_bf16(32, k, n, 10, std=0.01)
    say(f"fp8 7B gate {n}x{k}, m={m}")
    w8 = fr.fp8_quantize(f32_to_dev(w, dev))
    y = fr.fp8_lora_linear(bf16_to_dev(x, dev), w8, bf16_to_dev(a, dev), bf16_to_dev(b, dev), LORA_SCALE)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(m).choice(n, 256, replace=False))
    codes, s = fp8.quantize(w[rows])  # row scales are per row: a row subset quantises identically
    assert np.array_equal(w8.codes[rows.tolist()].cpu().numpy(), codes)
    ref = fp8.lora_linear(x, codes, s, a, b[rows], LORA_SCALE)
    err = rel_l2(bf16_to_f64(bf16_from_dev(y)[:, rows]), ref)
    say(f"  rel-L2 {err:.3e}")
    assert err <= REL_L2_TOL


def test_decode_workspace_reused_across_shapes():
    """One zero-filled workspace serves a sequence of decode shapes: the per-row-group counters
    return to zero after every call, so each result equals a call with a fresh workspace."""
    dev = device()
    shapes = [(8, 4608, 3584, 32), (3, 520, 1040, 5), (64, 4608, 3584, 16), (1, 96, 272, 0), (33, 4608, 3584, 32)]
    need = max(fr.fp8_lora_linear_workspace_bytes(m, n, k, r) for m, n, k, r in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for (m, n, k, r) in shapes:
        say(f"fp8 decode m={m} n={n} k={k} r={r}, shared workspace")
        w, x, a, b = _linear_case(m, n, k, r, seed=2 * m + n)
        w8 = fr.fp8_quantize(f32_to_dev(w, dev))
        xt = bf16_to_dev(x, dev)
        at = bf16_to_dev(a, dev) if r else None
        bt = bf16_to_dev(b, dev) if r else None
        y_shared = fr.fp8_lora_linear(xt, w8, at, bt, LORA_SCALE, workspace=ws)
        y_fresh = fr.fp8_lora_linear(xt, w8, at, bt, LORA_SCALE)
        torch.cuda.synchronize()
        assert torch.equal(y_shared, y_fresh)
