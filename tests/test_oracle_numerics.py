"""Pins of the oracle's bf16 rounding and rel-L2 (CPU only)."""
from fractions import Fraction

import numpy as np
import torch

from oracle.numerics import bf16_round, bf16_bits_of, bf16_to_f64, rel_l2


def _torch_bf16(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_bf16_round_matches_torch_on_float32_patterns():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # torch turns values beyond the bf16 range into inf as well
    ours = bf16_round(f.astype(np.float64))
    ref = _torch_bf16(f)
    assert np.array_equal(ours, ref, equal_nan=False)


def test_bf16_round_ties_and_subnormals():
    cases = np.array([
        1 + 2**-8,            # tie -> even (down)
        1 + 3 * 2**-8,        # tie -> even (up)
        1 + 2**-8 + 2**-30,   # just above tie -> up
        2**-133,              # smallest bf16 subnormal
        2**-134,              # tie with 0 -> 0
        3 * 2**-134,          # tie between 2^-133 and 2^-132 -> 2^-132
        -0.0,
        float.fromhex("0x1.fep127"),
        float.fromhex("0x1.ffp127"),   # tie at the top -> overflows to inf
    ])
    want = np.array([1.0, 1 + 2**-6, 1 + 2**-7, 2**-133, 0.0, 2**-132, -0.0,
                     float.fromhex("0x1.fep127"), np.inf])
    got = bf16_round(cases)
    assert np.array_equal(got, want)
    assert np.signbit(got[6])


def _exact_bf16(x: float) -> float:
    """Round-half-even to 8 significant bits, by exact rational arithmetic."""
    if x == 0:
        return x
    fx = Fraction(x)
    a = abs(fx)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    return float(r) if fx > 0 else -float(r)


def test_bf16_round_float64_against_exact_rounding():
    rng = np.random.default_rng(2)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
        rng.standard_normal(500) * 2.0 ** -128,
    ])
    got = bf16_round(vals)
    want = np.array([_exact_bf16(float(v)) for v in vals])
    assert np.array_equal(got, want)


def test_bits_roundtrip_and_rel_l2():
    rng = np.random.default_rng(3)
    v = bf16_round(rng.standard_normal(1000))
    assert np.array_equal(bf16_to_f64(bf16_bits_of(v)), v)
    assert rel_l2(v, v) == 0.0
    assert abs(rel_l2(np.array([3.0, 4.0]) * 1.001, np.array([3.0, 4.0])) - 1e-3) < 1e-12
