"""GPU parity of fp4rl_nvfp4_quantize: codes, scale bytes and tensor scale byte-exact vs the oracle."""
import os

import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr
from oracle import nvfp4
from workloads import (QWEN25_14B, bf16_bits, bf16_values, normal_f32, single_linear_config,
                       student_t3_weights, tensor_seed)

from gpu_util import assert_guards, bf16_to_dev, device, f32_to_dev, guarded, nvfp4_from_dev, say, tile_host
from test_oracle_nvfp4 import _load_golden

pytestmark = pytest.mark.gpu


def _gpu_quantize(w_np, dev, bf16=False, layout="row_major"):
    """Quantise on the GPU into guarded outputs (sentinel bytes around codes, scales and s_t, checked
    untouched) and download them as row-major arrays."""
    if bf16:
        wt = bf16_to_dev(bf16_bits(w_np), dev)
    else:
        wt = f32_to_dev(w_np, dev)
    n, k = w_np.shape
    lib = fr.load_library()
    lay = 1 if layout == "tiled" else 0
    cbuf, codes = guarded((lib.fp4rl_nvfp4_codes_bytes(n, k, lay),), torch.uint8, dev)
    sbuf, scales = guarded((lib.fp4rl_nvfp4_scales_bytes(n, k, lay),), torch.uint8, dev)
    tbuf, ts = guarded((1,), torch.float32, dev)
    out = fr.NVFP4Weight(codes, scales, ts, n, k, layout)
    fr.nvfp4_quantize(wt, layout=layout, out=out)
    torch.cuda.synchronize()
    for buf, what in ((cbuf, "codes"), (sbuf, "scales"), (tbuf, "tensor scale")):
        assert_guards(buf, f"quantiser {what} {n}x{k} {layout}")
    return nvfp4_from_dev(out)


def _assert_exact(got, want, what):
    c, s, t = got
    c0, s0, t0 = want
    assert np.float32(t).view(np.uint32) == np.float32(t0).view(np.uint32), f"{what}: s_t {t} vs {t0}"
    nbad_s = int(np.count_nonzero(s != s0))
    nbad_c = int(np.count_nonzero(c != c0))
    assert nbad_s == 0 and nbad_c == 0, f"{what}: {nbad_s} scale bytes, {nbad_c} code bytes differ"


def test_single_linear_weight_fp32():
    dev = device()
    cfg = single_linear_config(0)
    say("quantize 256x512 fp32 (seed 0)")
    _assert_exact(_gpu_quantize(cfg["w"], dev), nvfp4.quantize(cfg["w"]), "256x512")


def test_single_linear_weight_bf16_input():
    dev = device()
    w = single_linear_config(0)["w"]
    wb = bf16_values(bf16_bits(w))
    say("quantize 256x512 bf16")
    _assert_exact(_gpu_quantize(w, dev, bf16=True), nvfp4.quantize(wb), "256x512 bf16")


def test_golden_blocks(golden_dir):
    dev = device()
    w, codes, scales, st = _load_golden(os.path.join(golden_dir, "nvfp4_blocks.txt"))
    say("quantize golden blocks")
    _assert_exact(_gpu_quantize(w, dev), (codes, scales, st), "golden")


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (37, 80), (130, 272), (257, 1040), (2, 4096)])
def test_ragged_shapes(shape):
    dev = device()
    w = normal_f32(shape, 0.02, seed=shape[0] * 1000 + shape[1])
    say(f"quantize ragged {shape}")
    ref = nvfp4.quantize(w)
    _assert_exact(_gpu_quantize(w, dev), ref, str(shape))
    _assert_exact(_gpu_quantize(w, dev, layout="tiled"), ref, f"{shape} tiled")
    _assert_exact(_gpu_quantize(w, dev, bf16=True), nvfp4.quantize(bf16_values(bf16_bits(w))),
                  f"{shape} bf16")


def test_edge_values():
    dev = device()
    rng = np.random.default_rng(5)
    cases = {
        "zeros": np.zeros((4, 64), np.float32),
        "neg_zeros": -np.zeros((4, 64), np.float32),
        "tiny_amax": (rng.standard_normal((8, 64)) * 1e-38).astype(np.float32),
        "denormal": (rng.standard_normal((8, 64)) * 1e-42).astype(np.float32),
        "huge": (rng.standard_normal((8, 64)) * 1e37).astype(np.float32),
        "wide_range": (rng.standard_normal((16, 128)) * 10.0 ** rng.integers(-30, 30, (16, 128))).astype(np.float32),
        "one_outlier": np.where(np.arange(64 * 64).reshape(64, 64) == 77, 1e4,
                                rng.standard_normal((64, 64)) * 1e-3).astype(np.float32),
    }
    for name, w in cases.items():
        say(f"quantize edge case {name}")
        _assert_exact(_gpu_quantize(w, dev), nvfp4.quantize(w), name)


def _adversarial_weights():
    """Every row holds exact grid points, midpoints and their fp32 neighbours for its block scales."""
    rng = np.random.default_rng(6)
    n, k = 512, 256
    w = np.zeros((n, k), np.float32)
    w[0, 0] = 3.0  # tensor amax
    s_t = np.float32(np.float32(3.0) / np.float32(2688))
    mids = np.array([0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6.2, 6.375])
    for i in range(1, n):
        for b in range(k // 16):
            byte = int(rng.integers(1, 0x7F))
            d = np.float32(np.float32(nvfp4.e4m3_value(byte)) * s_t)
            pts = (mids * np.float64(d)).astype(np.float32)
            pick = rng.integers(0, 3, 16)
            vals = np.where(pick == 0, pts, np.where(pick == 1, np.nextafter(pts, np.float32(np.inf)),
                                                     np.nextafter(pts, np.float32(0))))
            vals = vals * np.where(rng.random(16) < 0.5, -1, 1)
            w[i, 16 * b:16 * b + 16] = vals.astype(np.float32)
    return w


def test_adversarial_midpoints():
    dev = device()
    w = _adversarial_weights()
    say("quantize adversarial midpoints 512x256")
    _assert_exact(_gpu_quantize(w, dev), nvfp4.quantize(w), "adversarial")


@pytest.mark.parametrize("name", ["qkv", "o", "gate", "up", "down"])
def test_full_size_14b_heavy_tailed(name):
    """Every 14B matrix shape, whole, Student-t(3) x0.02 with 1e-4 outliers x50, byte-exact."""
    dev = device()
    n, k = QWEN25_14B[name]
    w = student_t3_weights((n, k), tensor_seed(4, 0, name))
    say(f"quantize 14B {name} {n}x{k} full")
    _assert_exact(_gpu_quantize(w, dev), nvfp4.quantize(w), f"14B {name}")


def test_tiled_layout_and_repack():
    """The tiled quantiser output and the row-major -> tiled repack both equal the host permutation."""
    dev = device()
    # (33, 640): five chunks, so a second, partial region of tiles; (20, 1296):
    # a ragged last chunk in the eleventh tile column
    for n, k in [(1, 16), (37, 80), (48, 384), (130, 272), (33, 640), (20, 1296), (4608, 3584)]:
        w = normal_f32((n, k), 0.02, n + k)
        ref = nvfp4.quantize(w)
        wt = f32_to_dev(w, dev)
        tiled = fr.nvfp4_quantize(wt, layout="tiled")
        _assert_exact(nvfp4_from_dev(tiled), ref, f"tiled {n}x{k}")
        rm = fr.nvfp4_quantize(wt, layout="row_major")
        rep = fr.nvfp4_to_tiled(rm)
        torch.cuda.synchronize()
        ct, st = tile_host(ref[0], ref[1], n, k)
        assert np.array_equal(rep.codes.cpu().numpy(), ct) and np.array_equal(rep.scales.cpu().numpy(), st)
        assert np.array_equal(tiled.codes.cpu().numpy(), ct) and np.array_equal(tiled.scales.cpu().numpy(), st)


def test_tiled_bf16_input_ragged():
    """bf16 weights into the tiled layout, ragged in both dimensions, equal the host permutation."""
    dev = device()
    for n, k in [(21, 656), (300, 5120)]:
        w = normal_f32((n, k), 0.02, 3 * n + k)
        wb = bf16_bits(w)
        ref = nvfp4.quantize(bf16_values(wb))
        say(f"quantize bf16 {n}x{k} tiled")
        tiled = fr.nvfp4_quantize(bf16_to_dev(wb, dev), layout="tiled")
        torch.cuda.synchronize()
        ct, st = tile_host(ref[0], ref[1], n, k)
        assert np.array_equal(tiled.codes.cpu().numpy(), ct) and np.array_equal(tiled.scales.cpu().numpy(), st)
        assert np.float32(tiled.tensor_scale.cpu().numpy()[0]) == ref[2]


@pytest.mark.parametrize("layout", ["row_major", "tiled"])
def test_rounding_record(layout):
    """The rounding record (1 bit per element: rounded up in magnitude) is bit-exact, and the
    codes and scales of the recording call equal the plain quantiser's."""
    dev = device()
    rng = np.random.default_rng(12)
    cases = {
        "37x80": normal_f32((37, 80), 0.02, 37),
        "20x1296": normal_f32((20, 1296), 0.02, 20),
        "1024x2048": normal_f32((1024, 2048), 0.02, 1024),
        "adversarial": _adversarial_weights(),
        "wide_range": (rng.standard_normal((16, 128)) * 10.0 ** rng.integers(-30, 30, (16, 128))).astype(np.float32),
        "zeros": np.zeros((4, 64), np.float32),
    }
    for name, w in cases.items():
        for bf16 in (False, True):
            wr = bf16_values(bf16_bits(w)) if bf16 else w
            n, k = w.shape
            say(f"rounding record {name} {layout}{' bf16' if bf16 else ''}")
            wt = bf16_to_dev(bf16_bits(w), dev) if bf16 else f32_to_dev(w, dev)
            ru = torch.empty((n, k // 8), dtype=torch.uint8, device=dev)
            q = fr.nvfp4_quantize(wt, layout=layout, round_up=ru)
            torch.cuda.synchronize()
            _assert_exact(nvfp4_from_dev(q), nvfp4.quantize(wr), f"{name} record call")
            want = nvfp4.rounding_record(wr)
            got = ru.cpu().numpy()
            nbad = int(np.count_nonzero(got != want))
            assert nbad == 0, f"{name} {layout} bf16={bf16}: {nbad} record bytes differ"


def test_repeat_runs_identical():
    dev = device()
    w = f32_to_dev(normal_f32((1024, 2048), 0.02, 9), dev)
    a = nvfp4_from_dev(fr.nvfp4_quantize(w))
    b = nvfp4_from_dev(fr.nvfp4_quantize(w))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_empty_matrix_writes_zero_scale():
    dev = device()
    wq = fr.nvfp4_quantize(torch.empty((0, 32), dtype=torch.float32, device=dev), layout="row_major")
    torch.cuda.synchronize()
    assert float(wq.tensor_scale.cpu()[0]) == 0.0
