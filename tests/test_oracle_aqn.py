"""Pins of the oracle's AQN pieces: Philox words, normals, schedule, RMSNorm (CPU only)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch
from scipy import stats

from oracle import aqn
from oracle.numerics import bf16_round
from workloads import bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def torch_philox_exe():
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    d = tempfile.mkdtemp(prefix="philox_ref_")
    exe = os.path.join(d, "philox_ref")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc,
                    os.path.join(HERE, "philox_torch_ref.cpp"), "-o", exe], check=True)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def test_philox_words_match_torch_engine(torch_philox_exe):
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2**32, size=(300, 4), dtype=np.uint64)
    key = rng.integers(0, 2**32, size=(300, 2), dtype=np.uint64)
    ctr[0] = 0
    key[0] = 0
    ctr[1] = 0xFFFFFFFF
    key[1] = 0xFFFFFFFF
    lines = "\n".join(" ".join(str(int(v)) for v in (*c, *k)) for c, k in zip(ctr, key))
    out = subprocess.run([torch_philox_exe], input=lines, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    ref = np.array([[int(v) for v in ln.split()] for ln in out if ln.strip()], dtype=np.uint64)
    ours = np.stack([aqn.philox4x32_10(c[None, :], k)[0] for c, k in zip(ctr, key)])
    assert np.array_equal(ours.astype(np.uint64), ref)


def test_philox_counter_layout(torch_philox_exe):
    seed, step, norm_id = 0x1234567890ABCDEF, 0x00000007_00000003, 11
    words = aqn.philox_words(seed, step, norm_id, 5)
    lines = "\n".join(f"{q} {norm_id} {step & 0xFFFFFFFF} {step >> 32} "
                      f"{seed & 0xFFFFFFFF} {seed >> 32}" for q in range(5))
    out = subprocess.run([torch_philox_exe], input=lines, capture_output=True, text=True,
                         check=True).stdout.split()
    assert np.array_equal(words.ravel().astype(np.uint64), np.array(out, dtype=np.uint64))


def test_normals_are_standard_normal():
    z = aqn.philox_normal(seed=123, step=4, norm_id=2, d=1 << 20)
    assert abs(z.mean()) < 4 * 1 / np.sqrt(z.size)
    assert abs(z.var() - 1) < 4 * np.sqrt(2 / z.size)
    ks = stats.kstest(z, "norm")
    assert ks.pvalue > 1e-3
    # cos and sin halves are separately normal and uncorrelated
    zz = z.reshape(-1, 4)
    assert abs(np.corrcoef(zz[:, 0], zz[:, 1])[0, 1]) < 0.01
    assert stats.kstest(zz[:, 1], "norm").pvalue > 1e-3


def test_normals_depend_on_every_key_part():
    base = aqn.philox_normal(1, 2, 3, 64)
    for args in [(2, 2, 3), (1, 3, 3), (1, 2, 4), (1 << 40, 2, 3), (1, 2 | (1 << 33), 3)]:
        assert not np.allclose(aqn.philox_normal(*args, 64), base)
    assert np.array_equal(aqn.philox_normal(1, 2, 3, 64), base)
    # prefix property: a shorter draw is a prefix of a longer one
    assert np.array_equal(aqn.philox_normal(1, 2, 3, 10), base[:10])


def test_sigma_schedule_closed_form():
    s0, s1, kk = 1e-2, 5e-4, 10
    sig = np.array([aqn.sigma_schedule(s0, s1, k, kk) for k in range(kk)], dtype=np.float64)
    assert sig[0] == np.float32(s0) and sig[-1] == np.float32(s1)
    ratio = sig[1:] / sig[:-1]
    assert np.allclose(ratio, 0.05 ** (1 / 9), rtol=1e-6)
    assert np.all(np.diff(sig) < 0)            # large early, small late
    assert aqn.sigma_schedule(0.3, 0.1, 0, 1) == np.float32(0.3)
    with pytest.raises(ValueError):
        aqn.sigma_schedule(1, 1, 5, 5)


def test_sigma_zero_is_plain_rmsnorm():
    rng = np.random.default_rng(9)
    x = bf16_bits(rng.standard_normal((16, 512), dtype=np.float32))
    w = rng.uniform(0.5, 1.5, 512).astype(np.float32)
    y, wn = aqn.aqn_rmsnorm(x, w, 0.0, seed=1, step=0, norm_id=0, eps=1e-6)
    assert np.array_equal(wn, w.astype(np.float64))
    xt = torch.from_numpy((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (512,), weight=torch.from_numpy(w.astype(np.float64)),
                                       eps=float(np.float32(1e-6)))
    assert np.array_equal(y, bf16_round(ref.numpy()))


def test_noise_only_case_recovers_z():
    x = bf16_bits(np.ones((2, 300), dtype=np.float32))
    y, wn = aqn.aqn_rmsnorm(x, np.zeros(300, np.float32), 1.0, seed=3, step=1, norm_id=0, eps=0.0)
    z = aqn.philox_normal(3, 1, 0, 300)
    assert np.array_equal(wn, z)
    assert np.array_equal(y[0], bf16_round(z))


def test_sum_mode_equals_rescaled_mean_mode():
    rng = np.random.default_rng(10)
    x = bf16_bits(rng.standard_normal((4, 64), dtype=np.float32))
    w = rng.standard_normal(64)
    d, eps = 64, 1e-3
    a = aqn.rmsnorm_f64(x, w, eps, sum_mode=True)
    b = aqn.rmsnorm_f64(x, w / np.sqrt(d), np.float32(eps) / d, sum_mode=False)
    assert np.allclose(a, b, rtol=1e-12)


def test_golden_rows(golden_dir):
    with open(os.path.join(golden_dir, "rmsnorm_rows.txt")) as fh:
        for line in fh:
            if not line.startswith("case"):
                continue
            xs, ws, ys = line[4:].split("|")
            x = np.array([float(v) for v in xs.split()], dtype=np.float32)
            w = np.array([float(v) for v in ws.split()], dtype=np.float32)
            want = np.array([float(v) for v in ys.split()])
            y, _ = aqn.aqn_rmsnorm(bf16_bits(x[None, :]), w, 0.0, 0, 0, 0, eps=0.0)
            assert np.array_equal(y[0], want), line
