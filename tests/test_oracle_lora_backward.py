"""Pins of the oracle's LoRA backward (CPU only).

The backward is pinned against the forward oracle (itself pinned against
exact rationals) through adjoint identities, and against a term-by-term
Fraction evaluation on tiny shapes.
"""
import numpy as np

from oracle import linear, lora_backward as lb
from oracle.numerics import bf16_round
from oracle.nvfp4 import quantize
from workloads import bf16_bits, bf16_values, lora_bf16


def _case(seed, m, n, k, r, wscale=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * wscale).astype(np.float32)
    x = bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    dy = bf16_bits(rng.standard_normal((m, n), dtype=np.float32) * np.float32(0.1))
    a, b = lora_bf16(r, k, n, seed + 1, std=0.05)
    codes, scales, st = quantize(w)
    return dy, x, codes, scales, st, a, b


def test_float64_path_matches_exact_rationals():
    for seed, (m, n, k, r) in enumerate([(2, 3, 32, 2), (1, 4, 16, 1), (3, 2, 48, 3)]):
        dy, x, codes, scales, st, a, b = _case(seed, m, n, k, r)
        dx, da, db = lb.lora_linear_backward_f64(dy, x, codes, scales, st, a, b, 2.0)
        ex = lb.lora_backward_exact(dy, x, codes, scales, st, a, b, 2.0)
        for got, want in zip((dx, da, db), ex):
            w = np.array([[float(v) for v in row] for row in want])
            assert got.shape == w.shape
            assert np.allclose(got, w, rtol=1e-12, atol=1e-300)


def _ip(u, v):
    return float(np.sum(u * v))


def test_adjoint_identities_against_the_forward():
    """y is linear in x, and its LoRA term linear in A and in B separately:
    <dY, y(x + d) - y(x)> = <dX, d>, and likewise for the adapters."""
    m, n, k, r, s = 5, 48, 80, 4, 1.5
    dy, x, codes, scales, st, a, b = _case(30, m, n, k, r)
    dx, da, db = lb.lora_linear_backward_f64(dy, x, codes, scales, st, a, b, s)
    dyv = bf16_values(dy).astype(np.float64)
    rng = np.random.default_rng(31)
    fwd = (lambda xx, aa, bb: linear.lora_linear_f64(xx, codes, scales, st, aa, bb, s))
    y0 = fwd(x, a, b)
    d = bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    lhs = _ip(dyv, fwd(d, a, b))  # y(d) is the directional change for a linear map
    assert np.isclose(lhs, _ip(dx, bf16_values(d).astype(np.float64)), rtol=1e-10)
    da_dir = bf16_bits(rng.standard_normal((r, k), dtype=np.float32) * np.float32(0.05))
    lora_a = fwd(x, da_dir, b) - fwd(x, np.zeros_like(a), b)
    assert np.isclose(_ip(dyv, lora_a), _ip(da, bf16_values(da_dir).astype(np.float64)), rtol=1e-10)
    db_dir = bf16_bits(rng.standard_normal((n, r), dtype=np.float32) * np.float32(0.05))
    lora_b = fwd(x, a, db_dir) - fwd(x, a, np.zeros_like(b))
    assert np.isclose(_ip(dyv, lora_b), _ip(db, bf16_values(db_dir).astype(np.float64)), rtol=1e-10)
    # the forward's own value: <dY, y(x)> = <dX, x> only if the LoRA term is included in both
    assert np.isclose(_ip(dyv, y0), _ip(dx, bf16_values(x).astype(np.float64)), rtol=1e-10)


def test_reductions():
    dy, x, codes, scales, st, a, b = _case(32, 4, 32, 64, 3)
    base, na, nb = lb.lora_linear_backward_f64(dy, x, codes, scales, st)
    assert na is None and nb is None
    # s = 0: the adapter gradients vanish and dX is the base term alone
    dx0, da0, db0 = lb.lora_linear_backward_f64(dy, x, codes, scales, st, a, b, 0.0)
    assert np.array_equal(dx0, base) and not da0.any() and not db0.any()
    # zero weight: dX = s (dY B) A, checked column by column with plain sums
    zc, zs = np.zeros_like(codes), np.zeros_like(scales)
    dx, da, db = lb.lora_linear_backward_f64(dy, x, zc, zs, np.float32(0), a, b, 2.0)
    dyv, av, bv = (bf16_values(v).astype(np.float64) for v in (dy, a, b))
    for mm in range(4):
        for kk in (0, 17, 63):
            want = 2.0 * sum(sum(dyv[mm, i] * bv[i, j] for i in range(32)) * av[j, kk] for j in range(3))
            assert np.isclose(dx[mm, kk], want, rtol=1e-12)


def test_rounded_outputs_and_column_sampler():
    dy, x, codes, scales, st, a, b = _case(33, 6, 40, 96, 5)
    dx, da, db = lb.lora_linear_backward(dy, x, codes, scales, st, a, b, 2.0)
    dx64, da64, db64 = lb.lora_linear_backward_f64(dy, x, codes, scales, st, a, b, 2.0)
    assert np.array_equal(dx, bf16_round(dx64))
    assert np.array_equal(da, da64.astype(np.float32)) and np.array_equal(db, db64.astype(np.float32))
    h = 2.0 * bf16_values(dy).astype(np.float64) @ bf16_values(b).astype(np.float64)
    cols = np.array([0, 15, 16, 50, 95])
    assert np.allclose(lb.dx_columns_f64(dy, codes, scales, st, cols, a, h), dx64[:, cols], rtol=1e-12)


def test_adapter_terms_match_exact_rationals():
    """The weight-free (h, dA, dB-rows) form used for sampled checks at full size."""
    for seed, (m, n, k, r) in enumerate([(2, 3, 32, 2), (3, 5, 16, 4)]):
        dy, x, codes, scales, st, a, b = _case(40 + seed, m, n, k, r)
        _, da_ex, db_ex = lb.lora_backward_exact(dy, x, codes, scales, st, a, b, 2.0)
        rows = np.array([n - 1, 0])
        h, da, db = lb.adapter_terms_f64(dy, x, a, b, 2.0, b_rows=rows)
        da_w = np.array([[float(v) for v in row] for row in da_ex])
        db_w = np.array([[float(v) for v in row] for row in db_ex])
        assert np.allclose(da, da_w, rtol=1e-12, atol=1e-300)
        assert np.allclose(db, db_w[rows], rtol=1e-12, atol=1e-300)
        # h = s dY B, written out
        dyv, bv = bf16_values(dy).astype(np.float64), bf16_values(b).astype(np.float64)
        for mm in range(m):
            for j in range(r):
                assert np.isclose(h[mm, j], 2.0 * sum(dyv[mm, i] * bv[i, j] for i in range(n)), rtol=1e-12)
        _, _, db_all = lb.adapter_terms_f64(dy, x, a, b, 2.0)
        assert np.allclose(db_all, db_w, rtol=1e-12, atol=1e-300)


def test_backward_magnitudes():
    """On non-negative operands the magnitude sums are the backward's own results; elsewhere they bound them."""
    rng = np.random.default_rng(50)
    m, n, k, r = 4, 24, 48, 3
    pos = (lambda shape, sc: bf16_bits(np.abs(rng.standard_normal(shape, dtype=np.float32)) * np.float32(sc)))
    dy, x, a, b = pos((m, n), 0.1), pos((m, k), 1.0), pos((r, k), 0.05), pos((n, r), 0.05)
    codes, scales, st = quantize(np.abs(rng.standard_normal((n, k))).astype(np.float32) * np.float32(0.02))
    dxb, dxl, da_m, db_m = lb.backward_magnitudes_f64(dy, x, codes, scales, st, a, b, 2.0)
    dx, da, db = lb.lora_linear_backward_f64(dy, x, codes, scales, st, a, b, 2.0)
    assert np.allclose(dxb + dxl, dx, rtol=1e-13) and np.allclose(da_m, da, rtol=1e-13)
    assert np.allclose(db_m, db, rtol=1e-13)
    dy2, x2, c2, s2, t2, a2, b2 = _case(51, m, n, k, r)
    dxb, dxl, da_m, db_m = lb.backward_magnitudes_f64(dy2, x2, c2, s2, t2, a2, b2, -2.0)
    dx, da, db = lb.lora_linear_backward_f64(dy2, x2, c2, s2, t2, a2, b2, -2.0)
    assert np.all(np.abs(dx) <= (dxb + dxl) * (1 + 1e-12)) and np.all(np.abs(da) <= da_m * (1 + 1e-12))
    assert np.all(np.abs(db) <= db_m * (1 + 1e-12))
