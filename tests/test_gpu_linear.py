"""GPU parity of the fused W4A16 + LoRA linear (and its two halves) vs the oracle."""
import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr
from oracle import linear, nvfp4
from oracle.numerics import bf16_to_f64, rel_l2
from workloads import (LORA_SCALE, QWEN25_7B, QWEN25_32B, activations_bf16, bf16_bits, lora_bf16,
                       normal_f32, single_linear_config, tensor_seed)

from gpu_util import (REL_L2_TOL, accumulation_slack, assert_elementwise, assert_guards, bf16_from_dev, bf16_to_dev,
                      device, f32_to_dev, guarded, nvfp4_to_dev, say)

pytestmark = pytest.mark.gpu


def _case(m, n, k, r, seed, wstd=0.02, bstd=0.01, outliers=0.0):
    w = normal_f32((n, k), wstd, seed)
    x = activations_bf16(m, k, seed + 1, outlier_frac=outliers)
    a, b = lora_bf16(r, k, n, seed + 2, std=0.01)
    if bstd != 0.01:
        b = bf16_bits(normal_f32((n, r), bstd, seed + 3))
    return w, x, a, b


def _run(dev, x, q, a, b, s):
    """The fused linear into a guarded output (sentinel bytes on both sides, checked untouched)."""
    xt = bf16_to_dev(x, dev)
    wq = nvfp4_to_dev(*q, dev)
    at = bf16_to_dev(a, dev) if a is not None and a.shape[0] else None
    bt = bf16_to_dev(b, dev) if b is not None and b.shape[1] else None
    buf, y = guarded((x.shape[0], wq.n), torch.bfloat16, dev)
    fr.fp4_lora_linear(xt, wq, at, bt, s, out=y)
    torch.cuda.synchronize()
    assert_guards(buf, "linear output")
    return bf16_from_dev(y)


def _check(y_bits, y_ref, what, tol=REL_L2_TOL):
    err = rel_l2(bf16_to_f64(y_bits), y_ref)
    say(f"  {what}: rel-L2 {err:.3e}")
    assert err <= tol, f"{what}: rel-L2 {err}"


def _check_lin(y_bits, x, q, a, b, s, what, rows=None):
    """rel-L2 against the oracle, and every element within 2 bf16 ulps plus the fp32 accumulation bound
    derived from the magnitude of its terms."""
    ref = linear.lora_linear(x, *q, a, b, s, rows=rows)
    _check(y_bits, ref, what)
    base, lora = linear.lora_linear_magnitude_f64(x, *q, a, b, s, rows=rows)
    terms = x.shape[1] + (0 if a is None else np.asarray(a).shape[0])
    assert_elementwise(bf16_to_f64(y_bits), ref, accumulation_slack(base, lora, terms), what)


def test_single_linear_config():
    """W 256x512 ~N(0,.02), x 4x512, LoRA r=8 s=2, seed 0: GPU quantiser feeds the GPU linear."""
    dev = device()
    cfg = single_linear_config(0)
    q_ref = nvfp4.quantize(cfg["w"])
    wq = fr.nvfp4_quantize(f32_to_dev(cfg["w"], dev))
    y = fr.fp4_lora_linear(bf16_to_dev(cfg["x"], dev), wq, bf16_to_dev(cfg["lora_a"], dev),
                           bf16_to_dev(cfg["lora_b"], dev), cfg["lora_scale"])
    torch.cuda.synchronize()
    _check_lin(bf16_from_dev(y), cfg["x"], q_ref, cfg["lora_a"], cfg["lora_b"], cfg["lora_scale"], "256x512 M=4 r=8")


RAGGED = [  # (m, n, k, r)
    (1, 1, 16, 0), (1, 37, 48, 1), (3, 15, 144, 5), (16, 64, 128, 8), (17, 100, 512, 32),
    (33, 64, 160, 3), (64, 48, 256, 16), (65, 33, 96, 64), (127, 130, 384, 9), (128, 64, 512, 256),
    (129, 72, 208, 32), (300, 100, 1040, 24), (5, 4100, 32, 8),
]


@pytest.mark.parametrize("m,n,k,r", RAGGED)
def test_ragged_shapes(m, n, k, r):
    dev = device()
    w, x, a, b = _case(m, n, k, r, seed=m * 7919 + n * 31 + k)
    q = nvfp4.quantize(w)
    say(f"linear m={m} n={n} k={k} r={r}")
    y = _run(dev, x, q, a, b, LORA_SCALE)
    _check_lin(y, x, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r}")


SPLITK = [  # (m, n, k, r): few output tiles and a long K, so K is also split over workgroups
    (17, 40, 4096, 8), (20, 38, 4112, 4), (33, 100, 8192, 32), (64, 130, 6144, 16), (100, 72, 16384, 24),
    (128, 64, 12288, 64),
]


@pytest.mark.parametrize("m,n,k,r", SPLITK)
def test_split_k_shapes(m, n, k, r):
    dev = device()
    assert fr.fp4_linear_lora_up_workspace_bytes(m, n, k) > 0, "shape no longer splits K over workgroups"
    w, x, a, b = _case(m, n, k, r, seed=m * 131 + n * 17 + k)
    q = nvfp4.quantize(w)
    say(f"linear split-K m={m} n={n} k={k} r={r} ({fr.fp4_linear_kernel_name(m, n, k, r)})")
    y = _run(dev, x, q, a, b, LORA_SCALE)
    _check_lin(y, x, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r}")


SPLITK_CONFIGS = [  # (m, n, k, r, kernel): every split-K instantiation, ragged in n and k
    (33, 1000, 1040, 8, "splitk_kernel<2, 2, 4, 3>"),    # two row tiles per wave, three weight stages
    (64, 4600, 3568, 32, "splitk_kernel<2, 2, 4, 2>"),   # two row tiles, two stages (> 256 output tiles)
    (40, 9000, 3568, 16, "splitk_kernel<4, 2, 4, 2>"),   # four row tiles (wide), two stages
    (48, 700, 9232, 16, "splitk_kernel<4, 2, 4, 2>"),    # long K: four row tiles, K split over workgroups
]


@pytest.mark.parametrize("m,n,k,r,kernel", SPLITK_CONFIGS)
def test_split_k_launch_configs(m, n, k, r, kernel):
    dev = device()
    assert fr.fp4_linear_kernel_name(m, n, k, r) == kernel
    w, x, a, b = _case(m, n, k, r, seed=m * 97 + n * 13 + k)
    q = nvfp4.quantize(w)
    say(f"linear {kernel} m={m} n={n} k={k} r={r}")
    y = _run(dev, x, q, a, b, LORA_SCALE)
    _check_lin(y, x, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r}")


MID_CONFIGS = [  # (m, n, k, r): more than 96 tokens on at least 200 row groups of 128 features, or long K
    (100, 30000, 1040, 0),    # no adapters, a ragged last chunk
    (128, 30001, 272, 3),     # n % 4 != 0 (scalar stores), a short ragged K, r % 8 != 0 (scalar B loads)
    (97, 25601, 2064, 5),     # the fewest tokens, one feature past 200 row groups of 128
    (113, 26000, 3568, 32),   # tokens past M inside the last token group, a ragged K
    (128, 25473, 1040, 256),  # the largest rank: 128 tiles of t from the fused producers
    # fewer row groups and long K: the K split, fp32 partials and the finishing launch (t made separately)
    (113, 1001, 24592, 8),    # n % 4 != 0, a ragged last chunk, tokens past M in the last group
    (128, 300, 28672, 0),     # no adapters
    (97, 640, 24576, 100),    # a rank that is not a multiple of 8
]


@pytest.mark.parametrize("m,n,k,r", MID_CONFIGS)
def test_mid_kernel_configs(m, n, k, r):
    dev = device()
    kernel = fr.fp4_linear_kernel_name(m, n, k, r)
    assert kernel == "mid_kernel<1, 2, 4, 2, 3>"
    w, x, a, b = _case(m, n, k, r, seed=m * 89 + n * 11 + k)
    q = nvfp4.quantize(w)
    say(f"linear {kernel} m={m} n={n} k={k} r={r}")
    y = _run(dev, x, q, a, b, LORA_SCALE)
    _check_lin(y, x, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r}")


# a linear workspace starts with 5376 counter words: 1024 K-split tile counters,
# t tile counters, finished-tile count, 64 ready-flag lines of 256 bytes
COUNTER_BYTES = 4 * (1280 + 64 * 64)

FUSED = [  # (m, n, k, r): m <= 128 with r > 0 computes t inside the linear's launch, in K slices
    (1, 300, 4096, 32), (2, 100, 2048, 16), (1, 4608, 3584, 32), (8, 5000, 3584, 32), (13, 200, 1040, 7),
    (16, 18944, 3584, 32), (17, 64, 2048, 13), (33, 50, 1040, 7), (40, 300, 4096, 32), (100, 4608, 3584, 32),
    (128, 96, 4096, 256),
]


@pytest.mark.parametrize("m,n,k,r", FUSED)
def test_fused_lora_shapes(m, n, k, r):
    """Ragged ranks (scalar t loads), several K slices of t, and the most tiles of t (m = 128, r = 256)."""
    dev = device()
    w, x, a, b = _case(m, n, k, r, seed=m * 53 + n * 3 + k + r)
    q = nvfp4.quantize(w)
    say(f"linear fused LoRA m={m} n={n} k={k} r={r} ({fr.fp4_linear_kernel_name(m, n, k, r)})")
    xt, wq = bf16_to_dev(x, dev), nvfp4_to_dev(*q, dev)
    at, bt = bf16_to_dev(a, dev), bf16_to_dev(b, dev)
    ws = fr.linear_workspace(fr.fp4_lora_linear_workspace_bytes(m, n, k, r), dev)
    y1 = fr.fp4_lora_linear(xt, wq, at, bt, LORA_SCALE, workspace=ws)
    y2 = fr.fp4_lora_linear(xt, wq, at, bt, LORA_SCALE, workspace=ws)
    torch.cuda.synchronize()
    _check_lin(bf16_from_dev(y1), x, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r}")
    assert torch.equal(y1, y2), "second call on the same workspace differs"
    cb = COUNTER_BYTES
    assert not bool(ws[:cb].any()), "counter words not back at zero"
    # the producers leave t (all K slices added) in the first slice, right after the counters
    t_fused = ws[cb:cb + 4 * m * r].view(torch.float32).reshape(m, r).cpu().numpy()
    err = rel_l2(t_fused, linear.lora_down(x, a, LORA_SCALE))
    say(f"  t: rel-L2 {err:.3e}")
    assert err < 1e-5


@pytest.mark.parametrize("m", [1, 8, 40])
def test_lora_handoff_timeout_is_reported(m):
    """The bounded wait of the in-launch LoRA hand-off, made to give up from the host (the producers leave
    the ready flags down, the consumers poll 64 times): every kernel still ends, the workspace then reports
    FP4RL_ERR_TIMEOUT, also after a later normal call, until it is reset; after the reset a call matches
    the oracle and leaves the counter words at zero."""
    dev = device()
    n, k, r = 300, 1040, 16
    w, x, a, b = _case(m, n, k, r, seed=4242 + m)
    q = nvfp4.quantize(w)
    xt, wq = bf16_to_dev(x, dev), nvfp4_to_dev(*q, dev)
    at, bt = bf16_to_dev(a, dev), bf16_to_dev(b, dev)
    ws = fr.linear_workspace(fr.fp4_lora_linear_workspace_bytes(m, n, k, r), dev)
    say(f"linear hand-off timeout m={m} ({fr.fp4_linear_kernel_name(m, n, k, r)})")
    fr.linear_workspace_check(ws)  # a fresh workspace is healthy
    try:
        fr.debug_lora_handoff(64, True)
        fr.fp4_lora_linear(xt, wq, at, bt, LORA_SCALE, workspace=ws)
        torch.cuda.synchronize()
    finally:
        fr.debug_lora_handoff(0, False)
    with pytest.raises(fr.Fp4rlError) as err:
        fr.linear_workspace_check(ws)
    assert err.value.status == 9, err.value
    fr.fp4_lora_linear(xt, wq, at, bt, LORA_SCALE, workspace=ws)
    with pytest.raises(fr.Fp4rlError):
        fr.linear_workspace_check(ws)  # sticky until the counter words are cleared
    fr.linear_workspace_reset(ws)
    y = fr.fp4_lora_linear(xt, wq, at, bt, LORA_SCALE, workspace=ws)
    fr.linear_workspace_check(ws)
    _check_lin(bf16_from_dev(y), x, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r} after reset")
    assert not bool(ws[:COUNTER_BYTES].any()), "counter words not back at zero"


@pytest.mark.parametrize("m", [1, 8, 40])
def test_late_ready_flag_does_not_release_next_call(m):
    """Consumers made to give up after one poll while the producers still raise their ready flags, so a flag
    can go up after every consumer of its group has finished and cleared it. The next call on that workspace,
    made without a reset and on other tokens, still waits for its own producers (each call raises a ready
    value of its own) and matches the oracle; after a reset the counter words are back at zero."""
    dev = device()
    n, k, r = 300, 1040, 16
    w, x, a, b = _case(m, n, k, r, seed=5151 + m)
    x2 = activations_bf16(m, k, 5152 + m)
    q = nvfp4.quantize(w)
    wq, at, bt = nvfp4_to_dev(*q, dev), bf16_to_dev(a, dev), bf16_to_dev(b, dev)
    ws = fr.linear_workspace(fr.fp4_lora_linear_workspace_bytes(m, n, k, r), dev)
    say(f"linear late ready flag m={m} ({fr.fp4_linear_kernel_name(m, n, k, r)})")
    try:
        fr.debug_lora_handoff(1, False)
        fr.fp4_lora_linear(bf16_to_dev(x, dev), wq, at, bt, LORA_SCALE, workspace=ws)
        torch.cuda.synchronize()
    finally:
        fr.debug_lora_handoff(0, False)
    y = fr.fp4_lora_linear(bf16_to_dev(x2, dev), wq, at, bt, LORA_SCALE, workspace=ws)
    torch.cuda.synchronize()
    _check_lin(bf16_from_dev(y), x2, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r} after a late flag")
    fr.linear_workspace_reset(ws)
    fr.linear_workspace_check(ws)
    assert not bool(ws[:COUNTER_BYTES].any()), "counter words not back at zero"


PREFILL = [  # (m, n, k, r): more than 128 tokens (256- or 512-feature x 128-token workgroup tiles), ragged in
    # every dim; the last two take the eight-wave, 512-feature workgroups (at least 224 of them)
    (129, 16, 128, 0), (200, 270, 400, 8), (384, 512, 1024, 16), (1000, 520, 2064, 32), (2048, 300, 4096, 64),
    (4046, 3544, 1040, 24), (3970, 3600, 272, 0),
]


@pytest.mark.parametrize("m,n,k,r", PREFILL)
def test_prefill_shapes(m, n, k, r):
    dev = device()
    w, x, a, b = _case(m, n, k, r, seed=m * 13 + n * 7 + k, outliers=0.001)
    q = nvfp4.quantize(w)
    kernel = fr.fp4_linear_kernel_name(m, n, k, r)
    say(f"linear prefill m={m} n={n} k={k} r={r} ({kernel})")
    assert kernel == ("prefill_kernel<2, 8>" if m * n > 10**7 else "prefill_kernel<2, 4>")
    y = _run(dev, x, q, a, b, LORA_SCALE)
    _check_lin(y, x, q, a, b, LORA_SCALE, f"{m}x{n}x{k} r{r}")


def test_workspace_reuse_across_shapes():
    """One zero-filled workspace serves a sequence of split-K and plain calls, twice over: every result
    equals the result with a fresh workspace, bit for bit (the counters are back at zero after each call)."""
    dev = device()
    shapes = [(33, 100, 8192, 32), (64, 130, 6144, 16), (8, 96, 512, 8), (20, 38, 4112, 4)]
    cases = []
    for i, (m, n, k, r) in enumerate(shapes):
        w, x, a, b = _case(m, n, k, r, seed=900 + i)
        q = nvfp4.quantize(w)
        cases.append((bf16_to_dev(x, dev), nvfp4_to_dev(*q, dev), bf16_to_dev(a, dev), bf16_to_dev(b, dev)))
    big = max(fr.fp4_lora_linear_workspace_bytes(m, n, k, r) for m, n, k, r in shapes)
    shared = fr.linear_workspace(big, dev)
    fresh = [fr.fp4_lora_linear(*c, LORA_SCALE) for c in cases]
    for rep in range(2):
        for i, c in enumerate(cases):
            y = fr.fp4_lora_linear(*c, LORA_SCALE, workspace=shared)
            torch.cuda.synchronize()
            assert torch.equal(y, fresh[i]), f"pass {rep}, shape {shapes[i]}"
    say(f"  {len(shapes)} shapes x 2 passes on one workspace: identical")


def test_lora_reductions_bit_identical():
    dev = device()
    m, n, k, r = 24, 96, 256, 16
    w, x, a, b = _case(m, n, k, r, seed=42)
    q = nvfp4.quantize(w)
    base = _run(dev, x, q, None, None, 0.0)
    assert np.array_equal(_run(dev, x, q, a, np.zeros_like(b), LORA_SCALE), base), "B = 0"
    assert np.array_equal(_run(dev, x, q, a, b, 0.0), base), "s = 0"
    _check_lin(base, x, q, None, None, 0.0, "base only")


def test_lora_dominant():
    """W x1e-3 and B ~ N(0,1): the LoRA path carries most of y."""
    dev = device()
    m, n, k, r = 8, 256, 512, 32
    w, x, a, b = _case(m, n, k, r, seed=43, wstd=2e-5, bstd=1.0)
    q = nvfp4.quantize(w)
    y = _run(dev, x, q, a, b, LORA_SCALE)
    ref = linear.lora_linear(x, *q, a, b, LORA_SCALE)
    base = linear.lora_linear_f64(x, *q)
    assert np.linalg.norm(base) < 0.1 * np.linalg.norm(ref)
    _check_lin(y, x, q, a, b, LORA_SCALE, "LoRA-dominant")


def test_power_of_two_homogeneity_and_determinism():
    dev = device()
    m, n, k, r = 33, 200, 512, 8
    w, x, a, b = _case(m, n, k, r, seed=44)
    q = nvfp4.quantize(w)
    y1 = _run(dev, x, q, a, b, LORA_SCALE)
    x2 = bf16_bits(bf16_to_f64(x).astype(np.float32) * 2)
    y2 = _run(dev, x2, q, a, b, LORA_SCALE)
    assert np.array_equal(bf16_to_f64(y2), 2 * bf16_to_f64(y1))
    assert np.array_equal(_run(dev, x, q, a, b, LORA_SCALE), y1)


@pytest.mark.parametrize("m,r", [(40, 32), (100, 32), (300, 32), (200, 100), (129, 3)])
def test_halves_match_fused_call(m, r):
    """The two halves (lora_down, then the linear with t) against the one-call form; above 128 tokens t comes
    from the one-pass down-projection (every rank tile of 16 tokens per workgroup), ragged ranks included."""
    dev = device()
    n, k = 300, 640
    w, x, a, b = _case(m, n, k, r, seed=45)
    q = nvfp4.quantize(w)
    xt, wq = bf16_to_dev(x, dev), nvfp4_to_dev(*q, dev)
    at, bt = bf16_to_dev(a, dev), bf16_to_dev(b, dev)
    t = fr.lora_down(xt, at, LORA_SCALE)
    y_halves = fr.fp4_linear_lora_up(xt, wq, t, bt)
    y_fused = fr.fp4_lora_linear(xt, wq, at, bt, LORA_SCALE)
    torch.cuda.synchronize()
    # t is summed by differently shaped workgroups in the two calls (fp32
    # rounding order differs), so the outputs agree to bf16 rounding, and each
    # matches the oracle
    ref = linear.lora_linear(x, *q, a, b, LORA_SCALE)
    _check_lin(bf16_from_dev(y_halves), x, q, a, b, LORA_SCALE, "halves")
    _check_lin(bf16_from_dev(y_fused), x, q, a, b, LORA_SCALE, "fused")
    diff = (y_halves.float() - y_fused.float()).abs()
    assert float(diff.max()) <= 2.0 ** -7 * float(y_fused.float().abs().max())
    t_ref = linear.lora_down(x, a, LORA_SCALE)
    assert rel_l2(t.cpu().numpy(), t_ref) < 1e-5


def _full_size(dev, shapes, names, ms, r, config, outliers=0.0, sample=96):
    """Whole layer of linears; the GPU quantiser packs W, the oracle checks sampled output features."""
    rng = np.random.default_rng(config)
    for name in names:
        n, k = shapes[name]
        seed = tensor_seed(config, 0, name)
        w = normal_f32((n, k), 0.02, seed)
        wq = fr.nvfp4_quantize(f32_to_dev(w, dev))
        a, b = lora_bf16(r, k, n, seed + 17)
        at, bt = bf16_to_dev(a, dev), bf16_to_dev(b, dev)
        rows = np.sort(rng.choice(n, sample, replace=False))
        q_rows = nvfp4.quantize_rows(w, rows)
        for m in ms:
            x = activations_bf16(m, k, seed + m, outlier_frac=outliers)
            say(f"  {name} {n}x{k} M={m} r={r}")
            buf, y = guarded((m, n), torch.bfloat16, dev)
            fr.fp4_lora_linear(bf16_to_dev(x, dev), wq, at, bt, LORA_SCALE, out=y)
            torch.cuda.synchronize()
            assert_guards(buf, f"{name} M={m} output")
            y_rows = bf16_from_dev(y)[:, rows]
            _check_lin(y_rows, x, q_rows, a, b[rows], LORA_SCALE, f"{name} M={m}")
        del wq, w


def test_qwen7b_decode_layer():
    """7B layer linears at M = 1, 8, 32, 64, r = 32 (sampled output features)."""
    dev = device()
    _full_size(dev, QWEN25_7B, ["qkv", "o", "gate", "up", "down"], [1, 8, 32, 64], 32, config=1)


@pytest.mark.parametrize("name", ["qkv", "o", "gate", "up", "down"])
def test_qwen7b_prefill_outliers(name):
    """Each 7B linear at M = 8192 with 0.1% outlier channels x20 (sampled output features)."""
    dev = device()
    _full_size(dev, QWEN25_7B, [name], [8192], 32, config=2, outliers=0.001, sample=48)


def test_qwen32b_decode_m128():
    """32B layer linears at M = 128, r = 64 (sampled output features)."""
    dev = device()
    _full_size(dev, QWEN25_32B, ["qkv", "o", "gate", "up", "down"], [128], 64, config=3, sample=64)
