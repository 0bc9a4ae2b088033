"""GPU parity of the AQN RMSNorm and its Philox noise vs the oracle."""
import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr
from oracle import aqn
from oracle.numerics import bf16_round, bf16_to_f64, rel_l2
from workloads import activations_bf16, single_linear_config

from gpu_util import (REL_L2_TOL, assert_elementwise, assert_guards, bf16_from_dev, bf16_to_dev, device, f32_to_dev,
                      guarded, say)

pytestmark = pytest.mark.gpu


def _run(dev, x, w, sigma, seed, step, norm_id, eps, want_noise=True):
    """The norm into guarded outputs (sentinel bytes around y and w_noise, checked untouched)."""
    xt = bf16_to_dev(x, dev)
    wt = f32_to_dev(w, dev)
    ybuf, y = guarded(x.shape, torch.bfloat16, dev)
    wbuf, wn = guarded((w.shape[0],), torch.float32, dev) if want_noise else (None, None)
    fr.aqn_rmsnorm(xt, wt, sigma, seed, step, norm_id, eps, out=y, w_noise_out=wn)
    torch.cuda.synchronize()
    assert_guards(ybuf, f"AQN y {x.shape}")
    if want_noise:
        assert_guards(wbuf, f"AQN w_noise {w.shape}")
    return bf16_from_dev(y), (wn.cpu().numpy() if want_noise else None)


def _check(x, w, sigma, seed, step, norm_id, eps, dev, what, tol=REL_L2_TOL):
    y, wn = _run(dev, x, w, sigma, seed, step, norm_id, eps)
    y_ref, wn_ref = aqn.aqn_rmsnorm(x, w, sigma, seed, step, norm_id, eps)
    e_y = rel_l2(bf16_to_f64(y), y_ref)
    e_w = rel_l2(wn, wn_ref)
    say(f"  {what}: y rel-L2 {e_y:.3e}, w_noise rel-L2 {e_w:.3e}")
    assert e_y <= tol and e_w <= 1e-6, what
    # per element: the fp32 sum of d squares and the rsqrt bound the relative error by about
    # (d + 8) 2^-24, the noise's transcendental functions by 2^-20 of sigma |z| (inside |y| too)
    d = x.shape[1]
    slack = np.abs(y_ref) * ((d + 8) * 2.0 ** -24 + 2.0 ** -20)
    assert_elementwise(bf16_to_f64(y), y_ref, slack, f"{what} y")


def test_philox_words_bit_exact():
    dev = device()
    for seed, step, nid in [(0, 0, 0), (0x123456789ABCDEF, 7, 3), (2**64 - 1, 2**40 + 5, 2**32 - 1)]:
        got = fr.philox_words(seed, step, nid, 4096, dev).cpu().numpy().view(np.uint32)
        want = aqn.philox_words(seed, step, nid, 4096)
        assert np.array_equal(got, want), (seed, step, nid)


def test_single_linear_config_norm():
    dev = device()
    c = single_linear_config(0)
    _check(c["x"], c["norm_w"], c["sigma"], c["seed"], c["step"], c["norm_id"], c["eps"], dev, "4x512 s=1e-2")


def test_sigma_zero_is_plain_rmsnorm():
    dev = device()
    x = activations_bf16(64, 4096, 3)
    w = np.random.default_rng(3).uniform(0.5, 1.5, 4096).astype(np.float32)
    y, wn = _run(dev, x, w, 0.0, 1, 2, 3, 1e-6)
    assert np.array_equal(wn, w)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(bf16_to_f64(x)), (4096,),
                                       weight=torch.from_numpy(w.astype(np.float64)), eps=float(np.float32(1e-6)))
    e = rel_l2(bf16_to_f64(y), bf16_round(ref.numpy()))  # both sides rounded once to bf16
    say(f"  sigma=0 vs torch rms_norm: {e:.3e}")
    assert e <= REL_L2_TOL


def test_noise_only_exposes_z():
    """w = 0, sigma = 1: y = z * x / rms(x), so the noise itself is compared."""
    dev = device()
    x = activations_bf16(8, 5120, 4)
    _check(x, np.zeros(5120, np.float32), 1.0, 11, 3, 7, 1e-6, dev, "w=0 sigma=1")


@pytest.mark.parametrize("m,d", [(1, 1), (3, 7), (5, 100), (130, 513), (2, 4097), (17, 16384), (9, 8200),
                                 (1, 3584), (16, 264), (64, 5120), (256, 3584), (257, 3584)])
def test_ragged_shapes(m, d):
    dev = device()
    x = activations_bf16(m, d, m * 100 + d)
    w = np.random.default_rng(d).uniform(0.5, 1.5, d).astype(np.float32)
    _check(x, w, 1e-2, 5, 1, 2, 1e-6, dev, f"m={m} d={d}")


def test_few_rows_and_many_rows_paths_agree():
    """Up to 256 rows the columns are split over workgroups; beyond, one wave per row. Both sum the
    squares in the same order, so the first 256 rows of a 257-row batch equal the 256-row result."""
    dev = device()
    d = 3584
    x = activations_bf16(257, d, 77)
    w = np.random.default_rng(3).uniform(0.5, 1.5, d).astype(np.float32)
    y_many, wn_many = _run(dev, x, w, 1e-2, 5, 2, 1, 1e-6)
    y_few, wn_few = _run(dev, x[:256], w, 1e-2, 5, 2, 1, 1e-6)
    assert np.array_equal(y_many[:256], y_few) and np.array_equal(wn_many, wn_few)


def test_zero_rows_still_writes_noise():
    dev = device()
    w = np.ones(512, np.float32)
    wn = torch.empty(512, dtype=torch.float32, device=dev)
    fr.aqn_rmsnorm(torch.empty((0, 512), dtype=torch.bfloat16, device=dev), f32_to_dev(w, dev), 0.01, 9, 0, 0,
                   1e-6, w_noise_out=wn)
    torch.cuda.synchronize()
    assert rel_l2(wn.cpu().numpy(), aqn.noisy_weight(w, 0.01, 9, 0, 0)) < 1e-6


def test_qwen14b_stress_schedule():
    """65536 x 5120 bf16 tokens, sigma_k for k = 0..9 (Philox seed 4, step k): sampled rows per sigma."""
    dev = device()
    m, d = 65536, 5120
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    xt = torch.randn((m, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    w = np.ones(d, np.float32)
    wt = f32_to_dev(w, dev)
    rows = np.sort(np.random.default_rng(4).choice(m, 256, replace=False))
    x_rows = bf16_from_dev(xt[torch.from_numpy(rows).to(dev)])
    for k in range(10):
        sigma = fr.aqn_sigma(1e-2, 5e-4, k, 10)
        assert np.float32(sigma) == aqn.sigma_schedule(float(np.float32(1e-2)), float(np.float32(5e-4)), k, 10)
        wn = torch.empty(d, dtype=torch.float32, device=dev)
        y = fr.aqn_rmsnorm(xt, wt, sigma, 4, k, 0, 1e-6, w_noise_out=wn)
        torch.cuda.synchronize()
        y_rows = bf16_from_dev(y[torch.from_numpy(rows).to(dev)])
        ref, wn_ref = aqn.aqn_rmsnorm(x_rows, w, sigma, 4, k, 0, 1e-6)
        e = rel_l2(bf16_to_f64(y_rows), ref)
        say(f"  k={k} sigma={sigma:.4e}: y rel-L2 {e:.3e}")
        assert e <= REL_L2_TOL and rel_l2(wn.cpu().numpy(), wn_ref) < 1e-6
