"""Pins of the oracle's NVFP4 quantiser (CPU only).

Each pin comes from outside the oracle: torch's CPU float8_e4m3fn cast,
exact rational brute force over all 16 E2M1 codes, hand-worked golden blocks,
the format's error bound, and exact equivariances.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4
from oracle.nvfp4 import (quantize, dequantize, e4m3_encode, e4m3_value, unpack_codes,
                          tensor_scale)

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]


def _torch_e4m3(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


# ---------------------------------------------------------------- E4M3 ----

def test_e4m3_value_table_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = b.to(torch.float64).numpy()
    ours = e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def _e4m3_probe_values():
    """fp32 values around every E4M3 value and every midpoint, +- 40 ulps."""
    vals = e4m3_value(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    centres = np.concatenate([vals, mids, [464.0, 2.0 ** -10]]).astype(np.float32)
    bits = centres.view(np.uint32).astype(np.int64)
    offs = np.arange(-40, 41)
    nb = (bits[:, None] + offs[None, :]).ravel()
    nb = nb[(nb >= 0) & (nb < 0x7F800000)]
    return nb.astype(np.uint32).view(np.float32)


def test_e4m3_encode_matches_torch_near_every_boundary():
    f = _e4m3_probe_values()
    f = f[f <= 464.0]
    assert np.array_equal(e4m3_encode(f), _torch_e4m3(f))


def test_e4m3_encode_matches_torch_strided_sweep():
    # every 61st fp32 pattern in [0, 464]: ~18.7M values spanning all binades
    hi = np.float32(464.0).view(np.uint32)
    bits = np.arange(0, int(hi) + 1, 61, dtype=np.uint32)
    f = bits.view(np.float32)
    for chunk in np.array_split(f, 8):
        assert np.array_equal(e4m3_encode(chunk), _torch_e4m3(chunk))


def test_e4m3_encode_saturates():
    big = np.array([448.0, 449.0, 464.0, 464.5, 1e6, 3.4e38], dtype=np.float32)
    assert np.all(e4m3_encode(big) == 0x7E)


# ---------------------------------------------------------------- E2M1 ----

def _brute_force_codes(w32, d32):
    """Nearest signed E2M1 value over all 16 codes, in exact rationals.

    Tie-break: the even magnitude index; the sign bit is taken from x (IEEE
    keeps the sign of a value that rounds to zero).
    """
    x = Fraction(float(w32))
    d = Fraction(float(d32))
    best = None
    for code in range(16):
        mag = GRID[code & 7]
        val = -mag * d if code & 8 else mag * d
        dist = abs(x - val)
        key = (dist, (code & 7) % 2)
        if best is None or key < best[0]:
            best = (key, code)
    code = best[1]
    mag_idx = code & 7
    sign = 1 if np.signbit(np.float32(w32)) else 0
    if d == 0:
        mag_idx = 0
    return (sign << 3) | mag_idx


def _codes_of(w):
    packed, sbytes, s_t = quantize(w)
    return unpack_codes(packed), sbytes, s_t


@pytest.mark.parametrize("seed,k", [(0, 16), (1, 32), (2, 64)])
def test_e2m1_rounding_brute_force_random(seed, k):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((4, k)) * 0.02).astype(np.float32)
    c4, sbytes, s_t = _codes_of(w)
    for n in range(4):
        for kk in range(k):
            s_b = np.float32(e4m3_value(sbytes[n, kk // 16]))
            d = np.float32(s_b * s_t)
            assert c4[n, kk] == _brute_force_codes(w[n, kk], d), (n, kk)


def test_e2m1_rounding_brute_force_adversarial():
    """Grid points, midpoints and their fp32 neighbours, saturation, zeros."""
    rng = np.random.default_rng(7)
    rows = []
    for amax in [2.625, 1.0, 3.3e-3, 7.77]:
        for _ in range(3):
            s_t = np.float32(np.float32(amax) / np.float32(2688))
            # a block scale below the tensor one so D has a general mantissa
            d_guess = float(amax) / 6 * rng.uniform(0.05, 1.0)
            mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.2, 0.5, 3.0])
            pts = (mids * d_guess).astype(np.float32)
            nxt = np.nextafter(pts, np.float32(np.inf))
            prv = np.nextafter(pts, np.float32(0))
            vals = np.concatenate([pts, nxt, prv, [0.0, -0.0, 1e-30, -1e-30]])
            vals = vals * np.where(rng.random(vals.shape) < 0.5, -1, 1)
            vals = vals.astype(np.float32)
            blk = np.zeros(48, dtype=np.float32)
            blk[: len(vals)] = vals
            blk[47] = amax                        # pins the tensor amax
            rows.append(blk)
    w = np.stack(rows).astype(np.float32)
    c4, sbytes, s_t = _codes_of(w)
    n, k = w.shape
    for i in range(n):
        for kk in range(k):
            d = np.float32(np.float32(e4m3_value(sbytes[i, kk // 16])) * s_t)
            assert c4[i, kk] == _brute_force_codes(w[i, kk], d), (i, kk, w[i, kk])


def test_exact_midpoint_ties_go_to_even_index():
    # s_t = 2^-10, block scale 448, D = 0.4375: midpoints are exact fp32 numbers
    d = 0.4375
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * d
    blk = np.zeros(16, dtype=np.float32)
    blk[:7] = mids
    blk[15] = 2.625
    c4, sbytes, s_t = _codes_of(blk[None, :])
    assert s_t == np.float32(2.0 ** -10) and sbytes[0, 0] == 0x7E
    assert list(c4[0, :7]) == [0, 2, 2, 4, 4, 6, 6]


# ----------------------------------------------------- rounding record ----

def _record_bits(w):
    rec = nvfp4.rounding_record(w)
    return np.unpackbits(rec, axis=1, bitorder="little")


@pytest.mark.parametrize("seed,k", [(3, 16), (4, 48)])
def test_rounding_record_brute_force(seed, k):
    """The bit is 1 exactly when the brute-force nearest grid value exceeds |x| (rationals)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((4, k)) * 0.02).astype(np.float32)
    w[0, :4] = 0.0
    c4, sbytes, s_t = _codes_of(w)
    bits = _record_bits(w)
    for n in range(4):
        for kk in range(k):
            d = Fraction(float(np.float32(np.float32(e4m3_value(sbytes[n, kk // 16])) * s_t)))
            code = _brute_force_codes(w[n, kk], np.float32(float(d)))
            up = GRID[code & 7] * d > abs(Fraction(float(w[n, kk])))
            assert bits[n, kk] == int(up), (n, kk)


def test_rounding_record_closed_cases():
    """Exact grid points and saturated values round down (0); values just below a grid point
    that round to it round up (1); an all-zero block records 0."""
    d = 0.4375                                  # s_t = 2^-10, block byte 0x7E: D exact
    blk = np.zeros((2, 16), dtype=np.float32)
    grid = np.array([0.5, 1, 1.5, 2, 3, 4, 6]) * d
    blk[0, :7] = grid                           # exact grid points
    blk[0, 7:14] = np.nextafter(grid.astype(np.float32), np.float32(0))  # just below: up
    blk[0, 15] = 2.625                          # the amax (= 6 D): exact, down
    blk[1, :] = 0.0
    bits = _record_bits(blk)
    c4, sbytes, s_t = _codes_of(blk)
    assert s_t == np.float32(2.0 ** -10) and sbytes[0, 0] == 0x7E
    assert list(bits[0, :7]) == [0] * 7
    assert list(bits[0, 7:14]) == [1] * 7
    assert bits[0, 15] == 0 and not bits[1].any()
    # |x| beyond 6 D: block 1's r_b = 1.0625 ties to the E4M3 value 1.0 (even), so
    # D = 2^-10 and its max element sits at 6.375 D: saturated to 6 D, rounded down
    sat = np.zeros((1, 32), dtype=np.float32)
    sat[0, 0] = 2.625                           # tensor amax: s_t = 2^-10
    sat[0, 16] = np.float32(1.0625 * 6 * 2.0 ** -10)
    c4s, sb, st2 = _codes_of(sat)
    assert st2 == np.float32(2.0 ** -10) and sb[0, 1] == 0x38
    assert c4s[0, 16] & 7 == 7
    assert _record_bits(sat)[0, 16] == 0


def test_rounding_record_sign_symmetry_and_bound():
    """-W gives the same record; a 1 means the grid value exceeds |x| by at most half a step."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((8, 64)) * 0.02).astype(np.float32)
    assert np.array_equal(nvfp4.rounding_record(w), nvfp4.rounding_record(-w))
    packed, sbytes, s_t = quantize(w)
    deq = np.abs(dequantize(packed, sbytes, s_t))
    bits = _record_bits(w).astype(bool)
    # dequantize uses the exact S_b * s_t; the record uses fp32(S_b * s_t): they agree to 2^-24
    assert np.all(deq[bits] >= np.abs(w[bits]) * (1 - 2.0 ** -23))


# ------------------------------------------------------------- golden ----

def _load_golden(path):
    w, codes, scales, st = {}, {}, {}, None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *rest = line.split()
            if tag == "w":
                w[int(rest[0])] = [float.fromhex(v) if "x" in v else float(v) for v in rest[1:]]
            elif tag == "codes":
                codes[int(rest[0])] = [int(v, 16) for v in rest[1:]]
            elif tag == "scales":
                scales[int(rest[0])] = [int(v, 16) for v in rest[1:]]
            elif tag == "tensor_scale":
                st = float.fromhex(rest[0])
    n = len(w)
    return (np.array([w[i] for i in range(n)], dtype=np.float32),
            np.array([codes[i] for i in range(n)], dtype=np.uint8),
            np.array([scales[i] for i in range(n)], dtype=np.uint8), np.float32(st))


def test_golden_blocks(golden_dir):
    w, codes, scales, st = _load_golden(os.path.join(golden_dir, "nvfp4_blocks.txt"))
    packed, sbytes, s_t = quantize(w)
    assert s_t == st
    assert np.array_equal(sbytes, scales)
    assert np.array_equal(packed, codes)


# --------------------------------------------------- invariants / bounds ----

def test_tensor_scale_closed_form_and_amax_block():
    rng = np.random.default_rng(11)
    for _ in range(50):
        w = (rng.standard_normal((8, 64)) * rng.uniform(1e-3, 10)).astype(np.float32)
        packed, sbytes, s_t = quantize(w)
        amax = np.float32(np.abs(w).max())
        assert s_t == np.float32(amax / np.float32(2688.0))
        i, j = np.unravel_index(np.argmax(np.abs(w)), w.shape)
        assert sbytes[i, j // 16] == 0x7E
        assert (unpack_codes(packed)[i, j] & 7) == 7


def _step(q):
    return np.where(q <= 2, 0.5, np.where(q <= 4, 1.0, 2.0))


def test_error_bound_half_grid_step():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[3, 5] = 0.5      # an outlier makes many blocks use small / subnormal scales
    packed, sbytes, s_t = quantize(w)
    deq = dequantize(packed, sbytes, s_t)
    s_b = np.repeat(e4m3_value(sbytes), 16, axis=1)
    d = (s_b.astype(np.float32) * s_t).astype(np.float32).astype(np.float64)
    ax = np.abs(w.astype(np.float64))
    # the bound is stated against the encoder's D (fp32)
    g = np.abs(nvfp4.code_value(unpack_codes(packed)))
    err = np.abs(ax - g * d)
    normal = s_b >= 2.0 ** -6
    inside = ax <= 6 * d
    q = np.where(d > 0, ax / np.where(d > 0, d, 1), 0)
    bound = 0.5 * _step(np.minimum(q, 6.0)) * d
    sat = q > 6
    assert np.all(err[normal & ~sat] <= bound[normal & ~sat] * (1 + 1e-12))
    assert np.all(err[sat] <= 0.375 * d[sat] * (1 + 1e-12))
    sub = (~normal) & (d > 0)
    assert np.all(err[sub & inside] <= bound[sub & inside] * (1 + 1e-12))
    assert np.allclose(err[sub & ~inside], ax[sub & ~inside] - 6 * d[sub & ~inside])
    # dequantisation agrees with g * S_b * s_t within one fp32 rounding of D
    assert np.all(np.abs(np.abs(deq) - g * d) <= g * d * 2.0 ** -23)


def test_power_of_two_sign_and_permutation_equivariance():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    p, s, st = quantize(w)
    for e in (-5, 3, 17):
        p2, s2, st2 = quantize((w * np.float32(2.0 ** e)).astype(np.float32))
        assert np.array_equal(p, p2) and np.array_equal(s, s2)
        assert st2 == np.float32(st * np.float32(2.0 ** e))
    pn, sn, stn = quantize(-w)
    assert stn == st and np.array_equal(sn, s)
    c, cn = unpack_codes(p), unpack_codes(pn)
    assert np.array_equal(cn, c ^ 8)
    perm = rng.permutation(16)
    pp, sp, stp = quantize(w[perm])
    assert stp == st and np.array_equal(pp, p[perm]) and np.array_equal(sp, s[perm])
    bperm = rng.permutation(8)
    wb = w.reshape(16, 8, 16)[:, bperm].reshape(16, 128)
    pb, sb, _ = quantize(wb)
    assert np.array_equal(sb, s[:, bperm])
    assert np.array_equal(pb.reshape(16, 8, 8), p.reshape(16, 8, 8)[:, bperm])


def test_zero_tensor_and_nonfinite():
    z = np.zeros((2, 32), dtype=np.float32)
    z[1, 3] = -0.0
    p, s, st = quantize(z)
    assert st == 0 and not s.any()
    c = unpack_codes(p)
    assert c[1, 3] == 8 and (c & 7).max() == 0
    with pytest.raises(ValueError):
        tensor_scale(np.array([[1.0, np.inf]], dtype=np.float32))
    with pytest.raises(ValueError):
        quantize(np.zeros((2, 24), dtype=np.float32))


def test_quantize_rows_is_quantize_restricted():
    from oracle.nvfp4 import quantize_rows
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((50, 96)) * 0.02).astype(np.float32)
    w[7, 3] = 1.0
    p, s, st = quantize(w)
    rows = np.array([49, 7, 0, 21])
    p2, s2, st2 = quantize_rows(w, rows)
    assert st2 == st and np.array_equal(p2, p[rows]) and np.array_equal(s2, s[rows])
