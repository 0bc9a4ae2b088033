"""Helpers shared by the GPU parity tests (host <-> device marshalling only)."""
import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr

REL_L2_TOL = 1e-3  # bf16 outputs vs the bf16-rounded oracle (fp32 accumulate on the device)


def device():
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU visible")
    fr.load_library()  # raises if libfp4rl.so is missing: no silent fallback
    return torch.device("cuda:0")


def bf16_to_dev(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def bf16_from_dev(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_to_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def u8_to_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev)


def tile_host(codes, scales, n, k):
    """Row-major NVFP4 bytes -> the tiled layout (16-row x 128-k tiles), by index permutation.

    Tile (rt, c): 1024 code bytes ordered [g][i][j][4 B], word j of lane
    16 g + i = row 16 rt + i, bytes 64 c + 16 j + 4 g .. + 3 (k = 128 c + 32 j
    + 8 g .. + 7); 128 scale bytes ordered [p][i][j] = block 8 c + 2 j + p.
    """
    rt, kc = (n + 15) // 16, (k + 127) // 128
    cp = np.zeros((rt * 16, kc * 64), np.uint8)
    cp[:n, : k // 2] = codes
    sp = np.zeros((rt * 16, kc * 8), np.uint8)
    sp[:n, : k // 16] = scales
    # cp axes (rt, i, c, j, g, e) -> (rt, c, g, i, j, e); sp axes (rt, i, c, j, p) -> (rt, c, p, i, j)
    ct = cp.reshape(rt, 16, kc, 4, 4, 4).transpose(0, 2, 4, 1, 3, 5).reshape(-1)
    st = sp.reshape(rt, 16, kc, 4, 2).transpose(0, 2, 4, 1, 3).reshape(-1)
    return ct, st


def untile_host(ct, st, n, k):
    """Inverse of tile_host; also returns whether every padding byte is zero."""
    rt, kc = (n + 15) // 16, (k + 127) // 128
    cp = np.asarray(ct).reshape(rt, kc, 4, 16, 4, 4).transpose(0, 3, 1, 4, 2, 5).reshape(rt * 16, kc * 64)
    sp = np.asarray(st).reshape(rt, kc, 2, 16, 4).transpose(0, 3, 1, 4, 2).reshape(rt * 16, kc * 8)
    pad_zero = (not cp[n:].any() and not cp[:, k // 2:].any() and not sp[n:].any() and not sp[:, k // 16:].any())
    return cp[:n, : k // 2].copy(), sp[:n, : k // 16].copy(), pad_zero


def nvfp4_to_dev(codes, scales, s_t, dev) -> fr.NVFP4Weight:
    """Upload an oracle (row-major) NVFP4 matrix in the tiled layout the linear reads."""
    n, k = codes.shape[0], codes.shape[1] * 2
    ct, st = tile_host(codes, scales, n, k)
    return fr.NVFP4Weight(u8_to_dev(ct, dev), u8_to_dev(st, dev),
                          torch.tensor([np.float32(s_t)], dtype=torch.float32, device=dev), n, k, "tiled")


def nvfp4_from_dev(wq: fr.NVFP4Weight):
    """Download an NVFP4 matrix as row-major (codes [n, k/2], scales [n, k/16], s_t)."""
    torch.cuda.synchronize()
    c, s = wq.codes.cpu().numpy(), wq.scales.cpu().numpy()
    st = np.float32(wq.tensor_scale.cpu().numpy()[0])
    if wq.layout == "tiled":
        c, s, pad_zero = untile_host(c, s, wq.n, wq.k)
        assert pad_zero, "tiled padding is not zero"
        return c, s, st
    return c.reshape(wq.n, wq.k // 2), s.reshape(wq.n, wq.k // 16), st


def say(msg: str) -> None:
    print(msg, flush=True)


# ---------------------------------------------------------------- guard pads
GUARD_BYTES = 256   # sentinel bytes on each side of a guarded output
GUARD_FILL = 0x5A


def guarded(shape, dtype, dev):
    """An uninitialised-looking (sentinel-filled) contiguous output of `shape` inside a larger buffer with
    GUARD_BYTES of sentinel on each side; returns (buffer, view). The view stays 16-byte aligned."""
    elem = torch.empty((), dtype=dtype).element_size()
    nbytes = int(np.prod(shape)) * elem
    buf = torch.full((2 * GUARD_BYTES + nbytes,), GUARD_FILL, dtype=torch.uint8, device=dev)
    view = buf[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(tuple(shape))
    return buf, view


def assert_guards(buf, what=""):
    """The sentinel bytes on both sides of a guarded output are untouched (no out-of-bounds write)."""
    b = buf.cpu().numpy()
    lo, hi = b[:GUARD_BYTES], b[-GUARD_BYTES:]
    assert (lo == GUARD_FILL).all() and (hi == GUARD_FILL).all(), f"{what}: a write landed outside the output"


# ------------------------------------------------------- per-element bounds
def bf16_ulp(v):
    """Spacing of bf16 numbers in the binade of |v| (2^-133 below the normal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.maximum(a, 2.0 ** -126))  # a = f 2^e, f in [0.5, 1)
    return np.ldexp(1.0, e.astype(np.int64) - 1 - 7)


def f32_ulp(v):
    """Spacing of fp32 numbers at |v|."""
    return np.spacing(np.abs(np.asarray(v, dtype=np.float64)).astype(np.float32)).astype(np.float64)


def assert_elementwise(got, want, slack, what, ulp=bf16_ulp):
    """|got - want| <= 2 ulps of want (bf16 by default, or `ulp` = f32_ulp) + slack, element by element.

    The ulps cover the two roundings of the output (device and oracle); `slack`
    is the bound on the device's accumulation error the caller derives from
    the magnitude of the summed terms.
    """
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bound = 2.0 * ulp(want) + np.asarray(slack, dtype=np.float64)
    bad = np.argwhere(err > bound)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements beyond the per-element bound, first at {i}: "
                             f"got {got[i]!r} want {want[i]!r} bound {bound[i]!r}")
    worst = float(np.max(err / bound)) if err.size else 0.0
    say(f"  {what}: per-element error <= {worst:.3f} of the bound")


def accumulation_slack(base, lora, terms):
    """Bound on an fp32 accumulation of `terms` summands of total magnitude base + lora (each rounding
    contributes at most 2^-24 of the running magnitude), plus 2^-15 of the LoRA magnitude for its
    rank-space operand held as a bf16 hi + lo pair."""
    return (terms + 64) * 2.0 ** -24 * (np.asarray(base) + np.asarray(lora)) + 2.0 ** -15 * np.asarray(lora)
