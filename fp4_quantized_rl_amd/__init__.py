"""NVFP4 + LoRA + AQN rollout hot path for MI355X (gfx950).

Thin ctypes binding of ``libfp4rl.so`` (C ABI declared in include/fp4rl.h).
This module only marshals arguments: it checks dtype/shape/device/contiguity
of torch tensors, allocates outputs and workspaces with torch, and passes raw
device pointers plus torch's current HIP stream. Every step of the
computation runs in the library's HIP kernels. There is no CPU fallback: if
the library is not built, every call raises.

Operations (names follow the C ABI):
  nvfp4_quantize(w, layout[, round_up])     -> NVFP4Weight(codes, scales, tensor_scale) [+ rounding record]
  nvfp4_to_tiled(wq)                        -> row-major NVFP4 repacked into the tiled layout
  fp4_lora_linear(x, wq, lora_a, lora_b, s) -> y = x deq(Wq)^T + s (x A^T) B^T  (bf16)
  lora_down / fp4_linear_lora_up            -> the two halves of fp4_lora_linear
  fp4_lora_linear_backward(dy, x, wq, A, B, s) -> (dx bf16, dA fp32, dB fp32), the base frozen
  fp8_quantize(w) / fp8_lora_linear(x, w8, A, B, s, w8a8=False) -> FP8 (E4M3, per-row scale) rollout
  weights, W8A16 or W8A8 (per-token activation scales)
  fp4_gate_up_silu(x, wg, wu, (Ag, Bg), (Au, Bu), s) -> bf16(SiLU(x Wg^T + ...) * (x Wu^T + ...)), one launch
  aqn_sigma(s0, s1, k, K)                   -> exponential AQN noise level
  aqn_rmsnorm(x, w, sigma, seed, step, ...) -> RMSNorm with W_noise = w + sigma z
  philox_words(seed, step, norm_id, n)      -> raw Philox4x32-10 output blocks
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "LIB_PATH", "Fp4rlError", "load_library", "NVFP4Weight", "nvfp4_empty", "nvfp4_quantize", "nvfp4_to_tiled",
    "fp4_lora_linear", "fp4_lora_linear_backward", "fp4_lora_linear_backward_workspace_bytes",
    "FP8Weight", "fp8_quantize", "fp8_lora_linear", "fp8_lora_linear_workspace_bytes", "fp4_gate_up_silu",
    "fp4_gate_up_silu_workspace_bytes",
    "aqn_gate_up_silu", "aqn_lora_linear",
    "lora_down", "fp4_linear_lora_up", "fp4_linear_kernel_name", "linear_workspace",
    "fp4_lora_linear_workspace_bytes", "fp4_linear_lora_up_workspace_bytes", "aqn_sigma", "aqn_rmsnorm", "philox_words",
    "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4rl.so")

F32, BF16 = 0, 1
ROW_MAJOR, TILED = 0, 1
_LAYOUTS = {"row_major": ROW_MAJOR, "tiled": TILED}
_c = ctypes
_P = _c.c_void_p
_I64 = _c.c_int64
_STATUS = _c.c_int32

# name -> (restype, argtypes); must match include/fp4rl.h
_SIGNATURES = {
    "fp4rl_status_string": (_c.c_char_p, [_c.c_int32]),
    "fp4rl_last_error": (_c.c_char_p, []),
    "fp4rl_abi_version": (_c.c_int32, []),
    "fp4rl_nvfp4_quantize_workspace": (_c.c_size_t, [_I64, _I64]),
    "fp4rl_nvfp4_codes_bytes": (_c.c_size_t, [_I64, _I64, _c.c_int32]),
    "fp4rl_nvfp4_scales_bytes": (_c.c_size_t, [_I64, _I64, _c.c_int32]),
    "fp4rl_nvfp4_quantize": (_STATUS, [_P, _c.c_int32, _I64, _I64, _c.c_int32, _P, _P, _P, _P, _c.c_size_t, _P]),
    "fp4rl_nvfp4_to_tiled": (_STATUS, [_P, _P, _I64, _I64, _P, _P, _P]),
    "fp4rl_nvfp4_quantize_noalloc": (_STATUS, [_P, _c.c_int32, _I64, _I64, _c.c_int32, _P, _P, _P, _P]),
    "fp4rl_nvfp4_quantize_record": (_STATUS, [_P, _c.c_int32, _I64, _I64, _c.c_int32, _P, _P, _P, _P, _P,
                                              _c.c_size_t, _P]),
    "fp4rl_fp4_lora_linear_workspace": (_c.c_size_t, [_I64, _I64, _I64, _I64]),
    "fp4rl_fp4_lora_linear": (_STATUS, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _c.c_float, _P, _P,
                                        _c.c_size_t, _P]),
    "fp4rl_lora_down_workspace": (_c.c_size_t, [_I64, _I64, _I64]),
    "fp4rl_lora_down": (_STATUS, [_P, _I64, _I64, _P, _I64, _c.c_float, _P, _P, _c.c_size_t, _P]),
    "fp4rl_fp4_linear_lora_up_workspace": (_c.c_size_t, [_I64, _I64, _I64]),
    "fp4rl_fp4_linear_lora_up": (_STATUS, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _P, _P, _c.c_size_t,
                                           _P]),
    "fp4rl_fp4_linear_kernel_name": (_c.c_char_p, [_I64, _I64, _I64, _I64]),
    "fp4rl_linear_workspace_check": (_STATUS, [_P, _c.c_size_t, _P]),
    "fp4rl_linear_workspace_reset": (_STATUS, [_P, _c.c_size_t, _P]),
    "fp4rl_debug_lora_handoff": (None, [_c.c_uint32, _c.c_int32]),
    "fp4rl_fp4_gate_up_silu_workspace": (_c.c_size_t, [_I64, _I64, _I64, _I64]),
    "fp4rl_fp4_gate_up_silu": (_STATUS, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64,
                                         _c.c_float, _P, _P, _c.c_size_t, _P]),
    "fp4rl_aqn_gate_up_silu_workspace": (_c.c_size_t, [_I64, _I64, _I64, _I64]),
    "fp4rl_aqn_gate_up_silu": (_STATUS, [_P, _I64, _I64, _I64, _P, _c.c_float, _c.c_uint64, _c.c_uint64,
                                         _c.c_uint32, _c.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64,
                                         _c.c_float, _P, _P, _c.c_size_t, _P]),
    "fp4rl_aqn_lora_linear_workspace": (_c.c_size_t, [_I64, _I64, _I64, _I64]),
    "fp4rl_aqn_lora_linear": (_STATUS, [_P, _I64, _I64, _I64, _P, _c.c_float, _c.c_uint64, _c.c_uint64,
                                        _c.c_uint32, _c.c_float, _P, _P, _P, _P, _P, _I64, _c.c_float, _P, _P,
                                        _c.c_size_t, _P]),
    "fp4rl_fp8_quantize": (_STATUS, [_P, _c.c_int32, _I64, _I64, _P, _P, _P]),
    "fp4rl_fp8_lora_linear_workspace": (_c.c_size_t, [_I64, _I64, _I64, _I64]),
    "fp4rl_fp8_lora_linear": (_STATUS, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _I64, _c.c_float, _P, _P, _c.c_size_t,
                                        _P]),
    "fp4rl_fp8_lora_linear_w8a8_workspace": (_c.c_size_t, [_I64, _I64, _I64, _I64]),
    "fp4rl_fp8_lora_linear_w8a8": (_STATUS, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _I64, _c.c_float, _P, _P, _c.c_size_t,
                                        _P]),
    "fp4rl_fp4_lora_linear_backward_workspace": (_c.c_size_t, [_I64, _I64, _I64, _I64, _c.c_int32]),
    "fp4rl_fp4_lora_linear_backward": (_STATUS, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _c.c_float,
                                                 _P, _P, _P, _P, _c.c_size_t, _P]),
    "fp4rl_aqn_sigma": (_c.c_float, [_c.c_float, _c.c_float, _c.c_int32, _c.c_int32]),
    "fp4rl_aqn_rmsnorm": (_STATUS, [_P, _I64, _I64, _P, _c.c_float, _c.c_uint64, _c.c_uint64, _c.c_uint32,
                                    _c.c_float, _P, _P, _P]),
    "fp4rl_philox_words": (_STATUS, [_c.c_uint64, _c.c_uint64, _c.c_uint32, _I64, _P, _P]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_LIB = None


class Fp4rlError(RuntimeError):
    """A libfp4rl call returned a non-zero status (or the library is missing)."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(detail)


def load_library() -> ctypes.CDLL:
    """Load libfp4rl.so once; raises Fp4rlError if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise Fp4rlError(-1, f"{LIB_PATH} is missing: build it with "
                                 "`python -m fp4_quantized_rl_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(status: int, what: str) -> None:
    if status != 0:
        lib = load_library()
        name = lib.fp4rl_status_string(status).decode()
        detail = lib.fp4rl_last_error().decode()
        raise Fp4rlError(status, f"{what}: {name}: {detail}")


def _torch():
    import torch
    return torch


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev_tensor(t, name, dtypes, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


@dataclass
class NVFP4Weight:
    """An NVFP4 matrix [n, k]: flat uint8 codes and scales (layout "row_major" or
    "tiled", see include/fp4rl.h) and the fp32 tensor scale [1]."""

    codes: "object"
    scales: "object"
    tensor_scale: "object"
    n: int
    k: int
    layout: str = "tiled"

    @property
    def shape(self):
        return (self.n, self.k)

    @property
    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel() + 4

    def clone(self) -> "NVFP4Weight":
        return NVFP4Weight(self.codes.clone(), self.scales.clone(), self.tensor_scale.clone(), self.n, self.k,
                           self.layout)


def nvfp4_empty(n: int, k: int, layout: str = "tiled", device="cuda") -> NVFP4Weight:
    """Uninitialised NVFP4 storage for an [n, k] matrix in the given layout."""
    torch = _torch()
    lib = load_library()
    lay = _LAYOUTS[layout]
    cb = lib.fp4rl_nvfp4_codes_bytes(n, k, lay)
    sb = lib.fp4rl_nvfp4_scales_bytes(n, k, lay)
    return NVFP4Weight(torch.empty(max(cb, 16), dtype=torch.uint8, device=device)[:cb],
                       torch.empty(max(sb, 16), dtype=torch.uint8, device=device)[:sb],
                       torch.empty((1,), dtype=torch.float32, device=device), n, k, layout)


def nvfp4_quantize(w, layout: str = "tiled", out: NVFP4Weight | None = None, workspace=None,
                   round_up=None) -> NVFP4Weight:
    """NVFP4-quantise a [n, k] fp32 or bf16 weight (k % 16 == 0) on its device.

    round_up: optional uint8 [n, k // 8] device tensor that receives the
    rounding record (bit e of byte j: element 8 j + e rounded up in magnitude).
    """
    torch = _torch()
    _dev_tensor(w, "w", (torch.float32, torch.bfloat16), 2)
    n, k = w.shape
    if out is None:
        out = nvfp4_empty(n, k, layout, w.device)
    elif (out.n, out.k, out.layout) != (n, k, layout):
        raise ValueError("out does not match the weight shape / layout")
    lib = load_library()
    ws_bytes = lib.fp4rl_nvfp4_quantize_workspace(n, k)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=w.device)
    dt = F32 if w.dtype == torch.float32 else BF16
    with torch.cuda.device(w.device):
        if round_up is None:
            _check(lib.fp4rl_nvfp4_quantize(_ptr(w), dt, n, k, _LAYOUTS[layout], _ptr(out.codes), _ptr(out.scales),
                                            _ptr(out.tensor_scale), _ptr(workspace), workspace.numel(),
                                            _stream(w.device)),
                   "nvfp4_quantize")
        else:
            _dev_tensor(round_up, "round_up", (torch.uint8,), 2)
            if tuple(round_up.shape) != (n, k // 8) or round_up.device != w.device:
                raise ValueError("round_up must be uint8 [n, k // 8] on the weight's device")
            _check(lib.fp4rl_nvfp4_quantize_record(_ptr(w), dt, n, k, _LAYOUTS[layout], _ptr(out.codes),
                                                   _ptr(out.scales), _ptr(out.tensor_scale), _ptr(round_up),
                                                   _ptr(workspace), workspace.numel(), _stream(w.device)),
                   "nvfp4_quantize_record")
    return out


def nvfp4_to_tiled(wq: NVFP4Weight) -> NVFP4Weight:
    """Repack a row-major NVFP4 matrix into the tiled layout the linear kernels read."""
    torch = _torch()
    if wq.layout != "row_major":
        raise ValueError("expected a row_major NVFP4 weight")
    out = nvfp4_empty(wq.n, wq.k, "tiled", wq.codes.device)
    out.tensor_scale.copy_(wq.tensor_scale)
    with torch.cuda.device(wq.codes.device):
        _check(load_library().fp4rl_nvfp4_to_tiled(_ptr(wq.codes), _ptr(wq.scales), wq.n, wq.k, _ptr(out.codes),
                                                   _ptr(out.scales), _stream(wq.codes.device)),
               "nvfp4_to_tiled")
    return out


def _linear_args(x, wq: NVFP4Weight):
    torch = _torch()
    _dev_tensor(x, "x", (torch.bfloat16,), 2)
    _dev_tensor(wq.codes, "codes", (torch.uint8,))
    _dev_tensor(wq.scales, "scales", (torch.uint8,))
    _dev_tensor(wq.tensor_scale, "tensor_scale", (torch.float32,))
    if wq.layout != "tiled":
        raise ValueError("the linear kernels read the tiled NVFP4 layout (see nvfp4_to_tiled)")
    m, k = x.shape
    if wq.k != k:
        raise ValueError(f"x [{m},{k}] does not match the NVFP4 weight [{wq.n},{wq.k}]")
    return m, wq.n, k


def fp4_lora_linear(x, wq: NVFP4Weight, lora_a=None, lora_b=None, lora_scale: float = 0.0,
                    out=None, workspace=None):
    """y = bf16(x deq(Wq)^T + lora_scale (x A^T) B^T); x bf16 [m, k], A [r, k], B [n, r]."""
    torch = _torch()
    m, n, k = _linear_args(x, wq)
    r = 0
    if lora_a is not None or lora_b is not None:
        _dev_tensor(lora_a, "lora_a", (torch.bfloat16,), 2)
        _dev_tensor(lora_b, "lora_b", (torch.bfloat16,), 2)
        r = lora_a.shape[0]
        if lora_a.shape != (r, k) or lora_b.shape != (n, r):
            raise ValueError("LoRA shapes must be A [r, k] and B [n, r]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    ws_bytes = lib.fp4rl_fp4_lora_linear_workspace(m, n, k, r)
    if workspace is None and ws_bytes:
        workspace = linear_workspace(ws_bytes, x.device)
    with torch.cuda.device(x.device):
        _check(lib.fp4rl_fp4_lora_linear(_ptr(x), m, n, k, _ptr(wq.codes), _ptr(wq.scales),
                                         _ptr(wq.tensor_scale), _ptr(lora_a), _ptr(lora_b), r,
                                         float(lora_scale), _ptr(out), _ptr(workspace),
                                         0 if workspace is None else workspace.numel(),
                                         _stream(x.device)),
               "fp4_lora_linear")
    return out


def fp4_gate_up_silu_workspace_bytes(m: int, n: int, k: int, r: int) -> int:
    return load_library().fp4rl_fp4_gate_up_silu_workspace(m, n, k, r)


def fp4_gate_up_silu(x, wg: NVFP4Weight, wu: NVFP4Weight, lora_gate=None, lora_up=None, lora_scale: float = 0.0,
                     out=None, workspace=None):
    """h = bf16(SiLU(g) * u) for the NVFP4 + LoRA projections g (wg, lora_gate = (A, B)) and u of x [m <= 128, k].

    Up to 16 tokens one fused launch (g and u unrounded); from 17 tokens two
    linears whose bf16 outputs feed the gated product.
    """
    torch = _torch()
    m, n, k = _linear_args(x, wg)
    _linear_args(x, wu)
    if wu.n != n:
        raise ValueError("gate and up weights must have the same shape")
    r = 0
    ptrs = [None] * 4
    if lora_gate is not None or lora_up is not None:
        (ag, bg), (au, bu) = lora_gate, lora_up
        for t, nm in ((ag, "lora_a_gate"), (bg, "lora_b_gate"), (au, "lora_a_up"), (bu, "lora_b_up")):
            _dev_tensor(t, nm, (torch.bfloat16,), 2)
        r = ag.shape[0]
        if ag.shape != (r, k) or au.shape != (r, k) or bg.shape != (n, r) or bu.shape != (n, r):
            raise ValueError("LoRA shapes must be A [r, k] and B [n, r] for both projections")
        ptrs = [ag, bg, au, bu]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    need = lib.fp4rl_fp4_gate_up_silu_workspace(m, n, k, r)
    if workspace is None and need:
        # zero-filled: above 16 tokens it begins with a linear's counter words
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib.fp4rl_fp4_gate_up_silu(_ptr(x), m, n, k, _ptr(wg.codes), _ptr(wg.scales), _ptr(wg.tensor_scale),
                                          _ptr(wu.codes), _ptr(wu.scales), _ptr(wu.tensor_scale),
                                          *[_ptr(p) for p in ptrs], r, float(lora_scale), _ptr(out),
                                          _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                          _stream(x.device)), "fp4_gate_up_silu")
    return out


def aqn_gate_up_silu(x, norm_w, sigma: float, seed: int, step: int, norm_id: int, eps: float, wg: NVFP4Weight,
                     wu: NVFP4Weight, lora_gate=None, lora_up=None, lora_scale: float = 0.0, out=None,
                     workspace=None):
    """fp4_gate_up_silu of the AQN RMSNorm of x (raw bf16 [m <= 128, k]), the norm folded in (never stored)."""
    torch = _torch()
    m, n, k = _linear_args(x, wg)
    _linear_args(x, wu)
    _dev_tensor(norm_w, "norm_w", (torch.float32,), 1)
    if norm_w.shape[0] != k or wu.n != n:
        raise ValueError("norm_w must be [k] and the gate and up weights the same shape")
    r = 0
    ptrs = [None] * 4
    if lora_gate is not None or lora_up is not None:
        (ag, bg), (au, bu) = lora_gate, lora_up
        for t, nm in ((ag, "lora_a_gate"), (bg, "lora_b_gate"), (au, "lora_a_up"), (bu, "lora_b_up")):
            _dev_tensor(t, nm, (torch.bfloat16,), 2)
        r = ag.shape[0]
        if ag.shape != (r, k) or au.shape != (r, k) or bg.shape != (n, r) or bu.shape != (n, r):
            raise ValueError("LoRA shapes must be A [r, k] and B [n, r] for both projections")
        ptrs = [ag, bg, au, bu]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    need = lib.fp4rl_aqn_gate_up_silu_workspace(m, n, k, r)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib.fp4rl_aqn_gate_up_silu(_ptr(x), m, n, k, _ptr(norm_w), float(sigma), int(seed), int(step),
                                          int(norm_id), float(eps), _ptr(wg.codes), _ptr(wg.scales),
                                          _ptr(wg.tensor_scale), _ptr(wu.codes), _ptr(wu.scales),
                                          _ptr(wu.tensor_scale), *[_ptr(p) for p in ptrs], r, float(lora_scale),
                                          _ptr(out), _ptr(workspace), workspace.numel(), _stream(x.device)),
               "aqn_gate_up_silu")
    return out


def aqn_lora_linear(x, norm_w, sigma: float, seed: int, step: int, norm_id: int, eps: float, wq: NVFP4Weight,
                    lora_a=None, lora_b=None, lora_scale: float = 0.0, out=None, workspace=None):
    """fp4_lora_linear of the AQN RMSNorm of x (raw bf16 [m <= 128, k]), the norm folded in (never stored)."""
    torch = _torch()
    m, n, k = _linear_args(x, wq)
    _dev_tensor(norm_w, "norm_w", (torch.float32,), 1)
    if norm_w.shape[0] != k:
        raise ValueError("norm_w must be [k]")
    r = 0
    if lora_a is not None or lora_b is not None:
        _dev_tensor(lora_a, "lora_a", (torch.bfloat16,), 2)
        _dev_tensor(lora_b, "lora_b", (torch.bfloat16,), 2)
        r = lora_a.shape[0]
        if lora_a.shape != (r, k) or lora_b.shape != (n, r):
            raise ValueError("LoRA shapes must be A [r, k] and B [n, r]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    need = lib.fp4rl_aqn_lora_linear_workspace(m, n, k, r)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib.fp4rl_aqn_lora_linear(_ptr(x), m, n, k, _ptr(norm_w), float(sigma), int(seed), int(step),
                                         int(norm_id), float(eps), _ptr(wq.codes), _ptr(wq.scales),
                                         _ptr(wq.tensor_scale), _ptr(lora_a), _ptr(lora_b), r, float(lora_scale),
                                         _ptr(out), _ptr(workspace), workspace.numel(), _stream(x.device)),
               "aqn_lora_linear")
    return out


@dataclass
class FP8Weight:
    """E4M3 codes [n, k] (uint8) and fp32 row scales [n] on the device."""
    codes: object
    scales: object


def fp8_quantize(w) -> FP8Weight:
    """w fp32 or bf16 [n, k] -> FP8Weight (nearest E4M3 of w / s_n, s_n = amax_n / 448)."""
    torch = _torch()
    _dev_tensor(w, "w", (torch.float32, torch.bfloat16), 2)
    n, k = w.shape
    codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n,), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        _check(load_library().fp4rl_fp8_quantize(_ptr(w), BF16 if w.dtype == torch.bfloat16 else F32, n, k,
                                                 _ptr(codes), _ptr(scales), _stream(w.device)), "fp8_quantize")
    return FP8Weight(codes, scales)


def fp8_lora_linear_workspace_bytes(m: int, n: int, k: int, r: int, w8a8: bool = False) -> int:
    lib = load_library()
    if w8a8:
        return lib.fp4rl_fp8_lora_linear_w8a8_workspace(m, n, k, r)
    return lib.fp4rl_fp8_lora_linear_workspace(m, n, k, r)


def fp8_lora_linear(x, w8: FP8Weight, lora_a=None, lora_b=None, lora_scale: float = 0.0, out=None, workspace=None,
                    w8a8: bool = False):
    """y = bf16(x deq(W8)^T + lora_scale (x A^T) B^T); x bf16 [m, k].

    w8a8: quantise the tokens too (one E4M3 scale per row of x); the base product multiplies the E4M3 codes
    exactly (FP8 matrix cores, or widened to bf16 at 17..64 tokens); the LoRA term reads the bf16 x.
    """
    torch = _torch()
    _dev_tensor(x, "x", (torch.bfloat16,), 2)
    _dev_tensor(w8.codes, "codes", (torch.uint8,), 2)
    _dev_tensor(w8.scales, "scales", (torch.float32,), 1)
    m, k = x.shape
    n = w8.codes.shape[0]
    if w8.codes.shape[1] != k or w8.scales.shape[0] != n:
        raise ValueError("x [m, k], codes [n, k] and scales [n] do not match")
    r = 0
    if lora_a is not None or lora_b is not None:
        _dev_tensor(lora_a, "lora_a", (torch.bfloat16,), 2)
        _dev_tensor(lora_b, "lora_b", (torch.bfloat16,), 2)
        r = lora_a.shape[0]
        if lora_a.shape != (r, k) or lora_b.shape != (n, r):
            raise ValueError("LoRA shapes must be A [r, k] and B [n, r]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    need = fp8_lora_linear_workspace_bytes(m, n, k, r, w8a8)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    call, name = ((lib.fp4rl_fp8_lora_linear_w8a8, "fp8_lora_linear_w8a8") if w8a8
                  else (lib.fp4rl_fp8_lora_linear, "fp8_lora_linear"))
    with torch.cuda.device(x.device):
        _check(call(_ptr(x), m, n, k, _ptr(w8.codes), _ptr(w8.scales), _ptr(lora_a), _ptr(lora_b), r,
                    float(lora_scale), _ptr(out), _ptr(workspace), workspace.numel(), _stream(x.device)), name)
    return out


def fp4_lora_linear_backward_workspace_bytes(m: int, n: int, k: int, r: int, want_dx: bool = True) -> int:
    return load_library().fp4rl_fp4_lora_linear_backward_workspace(m, n, k, r, int(bool(want_dx)))


def fp4_lora_linear_backward(dy, x, wq: NVFP4Weight, lora_a=None, lora_b=None, lora_scale: float = 0.0,
                             want_dx: bool = True, workspace=None, out=None):
    """(dx, grad_a, grad_b) of y = x deq(Wq)^T + s (x A^T) B^T for dy bf16 [m, n].

    dx is bf16 [m, k] (None when want_dx is False); grad_a fp32 [r, k] and
    grad_b fp32 [n, r] (None without adapters). The base weight gets no gradient.
    out: optional (dx, grad_a, grad_b) tensors to write into (None entries are allocated).
    """
    torch = _torch()
    m, n, k = _linear_args(x, wq)
    _dev_tensor(dy, "dy", (torch.bfloat16,), 2)
    if dy.shape != (m, n):
        raise ValueError(f"dy must be [{m}, {n}]")
    r = 0
    if lora_a is not None or lora_b is not None:
        _dev_tensor(lora_a, "lora_a", (torch.bfloat16,), 2)
        _dev_tensor(lora_b, "lora_b", (torch.bfloat16,), 2)
        r = lora_a.shape[0]
        if lora_a.shape != (r, k) or lora_b.shape != (n, r):
            raise ValueError("LoRA shapes must be A [r, k] and B [n, r]")
    dev = x.device
    dx, ga, gb = out if out is not None else (None, None, None)
    if dx is None and want_dx:
        dx = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    if ga is None and r:
        ga = torch.empty((r, k), dtype=torch.float32, device=dev)
    if gb is None and r:
        gb = torch.empty((n, r), dtype=torch.float32, device=dev)
    if not want_dx:
        dx = None
    if not r:
        ga = gb = None
    for t, name, shape, dt in ((dx, "dx", (m, k), torch.bfloat16), (ga, "grad_a", (r, k), torch.float32),
                               (gb, "grad_b", (n, r), torch.float32)):
        if t is not None:
            _dev_tensor(t, name, (dt,), 2)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must be {list(shape)}")
    lib = load_library()
    ws_bytes = lib.fp4rl_fp4_lora_linear_backward_workspace(m, n, k, r, int(bool(want_dx)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(lib.fp4rl_fp4_lora_linear_backward(_ptr(dy), _ptr(x), m, n, k, _ptr(wq.codes), _ptr(wq.scales),
                                                  _ptr(wq.tensor_scale), _ptr(lora_a), _ptr(lora_b), r,
                                                  float(lora_scale), _ptr(dx), _ptr(ga), _ptr(gb), _ptr(workspace),
                                                  workspace.numel(), _stream(dev)),
               "fp4_lora_linear_backward")
    return dx, ga, gb


def lora_down(x, lora_a, lora_scale: float, out=None, workspace=None):
    """t = lora_scale * x A^T in fp32 [m, r]."""
    torch = _torch()
    _dev_tensor(x, "x", (torch.bfloat16,), 2)
    _dev_tensor(lora_a, "lora_a", (torch.bfloat16,), 2)
    m, k = x.shape
    r = lora_a.shape[0]
    if lora_a.shape[1] != k:
        raise ValueError("lora_a must be [r, k]")
    if out is None:
        out = torch.empty((m, r), dtype=torch.float32, device=x.device)
    lib = load_library()
    ws_bytes = lib.fp4rl_lora_down_workspace(m, k, r)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib.fp4rl_lora_down(_ptr(x), m, k, _ptr(lora_a), r, float(lora_scale), _ptr(out), _ptr(workspace),
                                   0 if workspace is None else workspace.numel(), _stream(x.device)), "lora_down")
    return out


def linear_workspace(nbytes: int, device="cuda"):
    """A zero-filled workspace for fp4_lora_linear / fp4_linear_lora_up (its counter words start at zero;
    the library returns them to zero after every call, so the buffer can be reused)."""
    return _torch().zeros(max(int(nbytes), 16), dtype=_torch().uint8, device=device)


def linear_workspace_check(workspace) -> None:
    """Synchronise the current stream and raise Fp4rlError (FP4RL_ERR_TIMEOUT) if a fused linear on this
    workspace gave up waiting for its in-launch LoRA producers."""
    if workspace is None:
        return
    torch = _torch()
    with torch.cuda.device(workspace.device):
        _check(load_library().fp4rl_linear_workspace_check(_ptr(workspace), workspace.numel(),
                                                           _stream(workspace.device)), "linear_workspace_check")


def linear_workspace_reset(workspace) -> None:
    """Zero the counter words of a linear workspace (a fill kernel on the current stream)."""
    if workspace is None:
        return
    torch = _torch()
    with torch.cuda.device(workspace.device):
        _check(load_library().fp4rl_linear_workspace_reset(_ptr(workspace), workspace.numel(),
                                                           _stream(workspace.device)), "linear_workspace_reset")


def debug_lora_handoff(spin_limit: int = 0, withhold_ready: bool = False) -> None:
    """Test hook: poll limit of the fused LoRA hand-off (0 = default) and whether producers withhold the flag."""
    load_library().fp4rl_debug_lora_handoff(int(spin_limit), 1 if withhold_ready else 0)


def fp4_lora_linear_workspace_bytes(m: int, n: int, k: int, r: int) -> int:
    return load_library().fp4rl_fp4_lora_linear_workspace(m, n, k, r)


def fp4_linear_lora_up_workspace_bytes(m: int, n: int, k: int) -> int:
    return load_library().fp4rl_fp4_linear_lora_up_workspace(m, n, k)


def fp4_linear_lora_up(x, wq: NVFP4Weight, t=None, lora_b=None, out=None, workspace=None):
    """y = bf16(s_t x deq^T + t B^T) with t fp32 [m, r] from lora_down (or None)."""
    torch = _torch()
    m, n, k = _linear_args(x, wq)
    r = 0
    if t is not None:
        _dev_tensor(t, "t", (torch.float32,), 2)
        _dev_tensor(lora_b, "lora_b", (torch.bfloat16,), 2)
        r = t.shape[1]
        if t.shape[0] != m or lora_b.shape != (n, r):
            raise ValueError("t must be [m, r] and lora_b [n, r]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    lib = load_library()
    ws_bytes = lib.fp4rl_fp4_linear_lora_up_workspace(m, n, k)
    if workspace is None and ws_bytes:
        workspace = linear_workspace(ws_bytes, x.device)
    with torch.cuda.device(x.device):
        _check(lib.fp4rl_fp4_linear_lora_up(_ptr(x), m, n, k, _ptr(wq.codes), _ptr(wq.scales),
                                            _ptr(wq.tensor_scale), _ptr(t), _ptr(lora_b), r, _ptr(out),
                                            _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                            _stream(x.device)),
               "fp4_linear_lora_up")
    return out


def fp4_linear_kernel_name(m: int, n: int, k: int, r: int = 0) -> str:
    """Main-kernel instantiation the library launches for an [m, k] x [n, k]^T product with rank r."""
    return load_library().fp4rl_fp4_linear_kernel_name(m, n, k, r).decode()


def aqn_sigma(sigma_start: float, sigma_end: float, k: int, num_stages: int) -> float:
    """sigma_k = sigma_start (sigma_end / sigma_start)^(k / (K - 1)); NaN for bad arguments."""
    return float(load_library().fp4rl_aqn_sigma(sigma_start, sigma_end, k, num_stages))


def aqn_rmsnorm(x, w, sigma: float, seed: int, step: int, norm_id: int, eps: float,
                out=None, w_noise_out=None):
    """bf16 RMSNorm of x [m, d] with the noisy weight w + sigma * PhiloxNormal(seed, step, norm_id)."""
    torch = _torch()
    _dev_tensor(x, "x", (torch.bfloat16,), 2)
    _dev_tensor(w, "w", (torch.float32,), 1)
    m, d = x.shape
    if w.shape[0] != d:
        raise ValueError("w must have length d")
    if w_noise_out is not None:
        _dev_tensor(w_noise_out, "w_noise_out", (torch.float32,), 1)
    if out is None:
        out = torch.empty_like(x)
    with torch.cuda.device(x.device):
        _check(load_library().fp4rl_aqn_rmsnorm(_ptr(x), m, d, _ptr(w), float(sigma), int(seed), int(step),
                                                int(norm_id), float(eps), _ptr(out), _ptr(w_noise_out),
                                                _stream(x.device)), "aqn_rmsnorm")
    return out


def philox_words(seed: int, step: int, norm_id: int, n_blocks: int, device="cuda"):
    """Raw Philox4x32-10 words of counter blocks 0..n_blocks-1: uint32 as int32 tensor [n_blocks, 4]."""
    torch = _torch()
    out = torch.empty((max(n_blocks, 1), 4), dtype=torch.int32, device=device)
    with torch.cuda.device(out.device):
        _check(load_library().fp4rl_philox_words(int(seed), int(step), int(norm_id), int(n_blocks), _ptr(out),
                                                 _stream(out.device)), "philox_words")
    return out[:n_blocks]
