"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import fp4_quantized_rl_amd as fr
from oracle import aqn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4rl.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_WORKSPACE, ERR_ARCH, ERR_HIP, ERR_VALUE = range(9)
FAKE = 0x7F0000000000   # 16-byte aligned, never dereferenced: every call below fails validation first
MIS = FAKE + 2          # misaligned


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4rl_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fr.LIB_PATH):
        from fp4_quantized_rl_amd.build import build
        build()
    return fr.load_library()


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(fr.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(fr.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name
    assert lib.fp4rl_abi_version() == 1


def test_status_strings(lib):
    names = [lib.fp4rl_status_string(i).decode() for i in range(10)]
    assert names[0] == "FP4RL_OK" and names[ERR_ALIGN] == "FP4RL_ERR_ALIGN"
    assert names[9] == "FP4RL_ERR_TIMEOUT"
    assert lib.fp4rl_status_string(99).decode() == "FP4RL_UNKNOWN_STATUS"


def test_quantize_rejects_bad_arguments(lib):
    def q(w, dt, n, k, c, s, ts, wsp, wsb, layout=1):
        return lib.fp4rl_nvfp4_quantize(w, dt, n, k, layout, c, s, ts, wsp, wsb, None)

    ws = lib.fp4rl_nvfp4_quantize_workspace(8, 32)
    assert ws >= 4
    assert q(FAKE, 0, 8, 24, FAKE, FAKE, FAKE, FAKE, ws) == ERR_SHAPE
    assert q(FAKE, 0, -1, 32, FAKE, FAKE, FAKE, FAKE, ws) == ERR_SHAPE
    assert q(FAKE, 7, 8, 32, FAKE, FAKE, FAKE, FAKE, ws) == ERR_DTYPE
    assert q(FAKE, 0, 8, 32, FAKE, FAKE, FAKE, FAKE, ws, layout=5) == ERR_VALUE
    assert q(None, 0, 8, 32, FAKE, FAKE, FAKE, FAKE, ws) == ERR_NULL
    assert q(FAKE, 0, 8, 32, FAKE, FAKE, None, FAKE, ws) == ERR_NULL
    assert q(FAKE, 0, 8, 32, FAKE, FAKE, FAKE, None, ws) == ERR_WORKSPACE
    assert q(FAKE, 0, 8, 32, FAKE, FAKE, FAKE, FAKE, ws - 1) == ERR_WORKSPACE
    assert q(MIS, 0, 8, 32, FAKE, FAKE, FAKE, FAKE, ws) == ERR_ALIGN
    assert q(FAKE, 0, 8, 32, FAKE, FAKE, FAKE + 1, FAKE, ws) == ERR_ALIGN
    assert lib.fp4rl_nvfp4_to_tiled(FAKE, FAKE, 8, 24, FAKE, FAKE, None) == ERR_SHAPE
    assert lib.fp4rl_nvfp4_to_tiled(FAKE, MIS, 8, 32, FAKE, FAKE, None) == ERR_ALIGN
    q(FAKE, 0, 8, 24, FAKE, FAKE, FAKE, FAKE, ws)
    assert "multiple of 16" in lib.fp4rl_last_error().decode()


def test_quantize_record_rejects_bad_arguments(lib):
    """The record entry point validates like fp4rl_nvfp4_quantize, and needs its round_up buffer."""
    def qr(w, n, k, ru, wsb, layout=1):
        return lib.fp4rl_nvfp4_quantize_record(w, 0, n, k, layout, FAKE, FAKE, FAKE, ru, FAKE, wsb, None)

    ws = lib.fp4rl_nvfp4_quantize_workspace(8, 32)
    assert qr(FAKE, 8, 32, None, ws) == ERR_NULL
    assert "round_up" in lib.fp4rl_last_error().decode()
    assert qr(FAKE, 8, 24, FAKE, ws) == ERR_SHAPE
    assert qr(MIS, 8, 32, FAKE, ws) == ERR_ALIGN
    assert qr(FAKE, 8, 32, FAKE, ws - 1) == ERR_WORKSPACE


def test_linear_rejects_bad_arguments(lib):
    f = lib.fp4rl_fp4_lora_linear
    ws = lib.fp4rl_fp4_lora_linear_workspace(4, 8, 32, 8)
    assert ws >= 4 * 8 * 4
    args = dict(x=FAKE, m=4, n=8, k=32, c=FAKE, s=FAKE, ts=FAKE, a=FAKE, b=FAKE, r=8, ls=2.0, y=FAKE,
                ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["m"], a["n"], a["k"], a["c"], a["s"], a["ts"], a["a"], a["b"], a["r"], a["ls"],
                 a["y"], a["ws"], a["wsb"], None)

    assert call(k=24) == ERR_SHAPE
    assert call(k=0) == ERR_SHAPE
    assert call(r=257) == ERR_SHAPE
    assert call(m=-1) == ERR_SHAPE
    assert call(m=1 << 20, k=1 << 11) == ERR_SHAPE     # m * k = 2^31: beyond 32-bit activation offsets
    assert call(m=16, k=1 << 26) == ERR_SHAPE          # 3..16 tokens: 2 m k bytes must stay below 2^31
    assert call(m=100, k=1 << 24) == ERR_SHAPE         # 17..128 tokens (split-K, mid-batch kernels): the same
    assert call(ls=float("nan")) == ERR_VALUE
    assert call(a=None) == ERR_NULL
    assert call(x=None) == ERR_NULL
    assert call(wsb=ws - 1) == ERR_WORKSPACE
    assert call(ws=None) == ERR_WORKSPACE
    assert call(y=MIS) == ERR_ALIGN
    assert call(ts=FAKE + 2) == ERR_ALIGN
    assert call(m=0) == OK and call(n=0) == OK          # empty: no-op, nothing touched
    assert lib.fp4rl_lora_down(FAKE, 4, 24, FAKE, 8, 1.0, FAKE, FAKE, 1 << 20, None) == ERR_SHAPE
    assert lib.fp4rl_lora_down(FAKE, 4, 32, FAKE, 0, 1.0, FAKE, None, 0, None) == OK
    need = lib.fp4rl_lora_down_workspace(1, 3584, 32)
    assert need >= 7 * 32 * 4
    assert lib.fp4rl_lora_down(FAKE, 1, 3584, FAKE, 32, 1.0, FAKE, FAKE, need - 1, None) == ERR_WORKSPACE
    assert lib.fp4rl_lora_down_workspace(8192, 3584, 32) == 0
    assert lib.fp4rl_fp4_linear_lora_up(FAKE, 4, 8, 32, FAKE, FAKE, FAKE, None, FAKE, 8, FAKE, None, 0,
                                        None) == ERR_NULL
    # K split over workgroups (decode-shaped m, few output tiles): fp32 partials + counters
    need = lib.fp4rl_fp4_linear_lora_up_workspace(64, 3584, 18944)
    assert need >= 2 * 64 * 3584 * 4
    assert lib.fp4rl_fp4_linear_lora_up(FAKE, 64, 3584, 18944, FAKE, FAKE, FAKE, None, None, 0, FAKE, FAKE, need - 1,
                                        None) == ERR_WORKSPACE
    assert lib.fp4rl_fp4_linear_lora_up_workspace(1, 3584, 18944) == 0
    assert (lib.fp4rl_fp4_lora_linear_workspace(64, 3584, 18944, 32)
            >= lib.fp4rl_fp4_linear_lora_up_workspace(64, 3584, 18944) + 64 * 32 * 4)


def test_backward_rejects_bad_arguments(lib):
    f = lib.fp4rl_fp4_lora_linear_backward
    ws = lib.fp4rl_fp4_lora_linear_backward_workspace(4, 8, 32, 8, 1)
    # Wt [k][n] bf16, Bt, At2, t, h, hs: each region 256-byte aligned
    assert ws >= 32 * 8 * 2 + 8 * 8 * 2 + 32 * 16 * 2 + 2 * 4 * 8 * 4 + 4 * 16 * 2
    assert lib.fp4rl_fp4_lora_linear_backward_workspace(4, 8, 32, 8, 0) < ws
    assert lib.fp4rl_fp4_lora_linear_backward_workspace(4, 12, 32, 8, 1) == 0  # n % 8 != 0: invalid
    args = dict(dy=FAKE, x=FAKE, m=4, n=8, k=32, c=FAKE, s=FAKE, ts=FAKE, a=FAKE, b=FAKE, r=8, ls=2.0, dx=FAKE,
                ga=FAKE, gb=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["dy"], a["x"], a["m"], a["n"], a["k"], a["c"], a["s"], a["ts"], a["a"], a["b"], a["r"], a["ls"],
                 a["dx"], a["ga"], a["gb"], a["ws"], a["wsb"], None)

    assert call(k=24) == ERR_SHAPE
    assert call(n=12) == ERR_SHAPE
    assert call(r=257) == ERR_SHAPE
    assert call(k=1 << 22) == ERR_SHAPE
    assert call(ls=float("inf")) == ERR_VALUE
    assert call(a=None) == ERR_NULL
    assert call(a=None, b=None, dx=None) == ERR_NULL     # nothing to compute
    assert call(ga=None) == ERR_NULL
    assert call(dy=None) == ERR_NULL
    assert call(x=None) == ERR_NULL
    assert call(c=None) == ERR_NULL
    assert call(dx=MIS) == ERR_ALIGN
    assert call(gb=MIS) == ERR_ALIGN
    assert call(wsb=ws - 1) == ERR_WORKSPACE
    assert call(ws=None) == ERR_WORKSPACE
    assert call(ws=FAKE + 16) == ERR_ALIGN
    assert call(m=0, n=0) == OK
    # x and the weight are not read when they are not needed
    assert call(a=None, b=None, x=None, ga=None, gb=None, wsb=lib.fp4rl_fp4_lora_linear_backward_workspace(
        4, 8, 32, 0, 1)) == ERR_HIP


def test_fp8_rejects_bad_arguments(lib):
    q = lib.fp4rl_fp8_quantize
    assert q(FAKE, 0, 8, 24, FAKE, FAKE, None) == ERR_SHAPE
    assert q(FAKE, 0, 8, 0, FAKE, FAKE, None) == ERR_SHAPE
    assert q(FAKE, 5, 8, 32, FAKE, FAKE, None) == ERR_DTYPE
    assert q(None, 0, 8, 32, FAKE, FAKE, None) == ERR_NULL
    assert q(MIS, 0, 8, 32, FAKE, FAKE, None) == ERR_ALIGN
    assert q(FAKE, 0, 0, 32, None, None, None) == OK
    f = lib.fp4rl_fp8_lora_linear
    ws = lib.fp4rl_fp8_lora_linear_workspace(4, 8, 32, 8)
    assert ws >= 4 * 8 * 4 + 4 * 8 * 4
    args = dict(x=FAKE, m=4, n=8, k=32, c=FAKE, s=FAKE, a=FAKE, b=FAKE, r=8, ls=2.0, y=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["m"], a["n"], a["k"], a["c"], a["s"], a["a"], a["b"], a["r"], a["ls"], a["y"], a["ws"],
                 a["wsb"], None)

    assert call(k=24) == ERR_SHAPE
    assert call(r=257) == ERR_SHAPE
    assert call(ls=float("nan")) == ERR_VALUE
    assert call(a=None) == ERR_NULL
    assert call(c=None) == ERR_NULL
    assert call(y=MIS) == ERR_ALIGN
    assert call(wsb=ws - 1) == ERR_WORKSPACE
    assert call(ws=FAKE + 16) == ERR_ALIGN
    assert call(m=0) == OK and call(n=0) == OK


def test_gate_up_rejects_bad_arguments(lib):
    f = lib.fp4rl_fp4_gate_up_silu
    ws = lib.fp4rl_fp4_gate_up_silu_workspace(4, 8, 32, 8)
    assert ws >= 2 * 4 * 8 * 4
    assert lib.fp4rl_fp4_gate_up_silu_workspace(129, 8, 32, 8) == 0
    args = dict(x=FAKE, m=4, n=8, k=32, gc=FAKE, gs=FAKE, gt=FAKE, uc=FAKE, us=FAKE, ut=FAKE, ag=FAKE, bg=FAKE,
                au=FAKE, bu=FAKE, r=8, ls=2.0, h=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["m"], a["n"], a["k"], a["gc"], a["gs"], a["gt"], a["uc"], a["us"], a["ut"], a["ag"],
                 a["bg"], a["au"], a["bu"], a["r"], a["ls"], a["h"], a["ws"], a["wsb"], None)

    assert call(m=129) == ERR_SHAPE
    assert call(k=24) == ERR_SHAPE
    assert call(r=257) == ERR_SHAPE
    assert call(ls=float("nan")) == ERR_VALUE
    assert call(au=None) == ERR_NULL
    assert call(uc=None) == ERR_NULL
    assert call(h=MIS) == ERR_ALIGN
    assert call(ut=FAKE + 2) == ERR_ALIGN
    assert call(wsb=ws - 1) == ERR_WORKSPACE
    assert call(m=0) == OK and call(n=0) == OK


def test_aqn_gate_up_rejects_bad_arguments(lib):
    f = lib.fp4rl_aqn_gate_up_silu
    ws = lib.fp4rl_aqn_gate_up_silu_workspace(4, 8, 32, 8)
    assert ws >= 32 * 4 + 4 * 4 + 2 * 4 * 8 * 4
    assert lib.fp4rl_aqn_gate_up_silu_workspace(4, 8, 32768, 8) == 0  # wider than the norm
    args = dict(x=FAKE, m=4, n=8, k=32, w=FAKE, sg=1e-2, seed=1, step=0, nid=0, eps=1e-6, gc=FAKE, gs=FAKE,
                gt=FAKE, uc=FAKE, us=FAKE, ut=FAKE, ag=FAKE, bg=FAKE, au=FAKE, bu=FAKE, r=8, ls=2.0, h=FAKE, ws=FAKE,
                wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["m"], a["n"], a["k"], a["w"], a["sg"], a["seed"], a["step"], a["nid"], a["eps"], a["gc"],
                 a["gs"], a["gt"], a["uc"], a["us"], a["ut"], a["ag"], a["bg"], a["au"], a["bu"], a["r"], a["ls"],
                 a["h"], a["ws"], a["wsb"], None)

    assert call(m=129) == ERR_SHAPE
    assert call(k=32768) == ERR_SHAPE
    assert call(sg=-1.0) == ERR_VALUE
    assert call(eps=float("nan")) == ERR_VALUE
    assert call(w=None) == ERR_NULL
    assert call(bu=None) == ERR_NULL
    assert call(w=MIS) == ERR_ALIGN
    assert call(wsb=ws - 1) == ERR_WORKSPACE
    assert call(ws=None) == ERR_WORKSPACE
    assert call(m=0) == OK


def test_aqn_lora_linear_rejects_bad_arguments(lib):
    f = lib.fp4rl_aqn_lora_linear
    ws = lib.fp4rl_aqn_lora_linear_workspace(4, 8, 32, 8)
    assert ws >= 32 * 4 + 4 * 4 + 4 * 8 * 4
    assert lib.fp4rl_aqn_lora_linear_workspace(4, 8, 32768, 8) == 0  # wider than the norm
    assert lib.fp4rl_aqn_lora_linear_workspace(129, 8, 32, 8) == 0   # more tokens than one launch takes
    args = dict(x=FAKE, m=4, n=8, k=32, w=FAKE, sg=1e-2, seed=1, step=0, nid=0, eps=1e-6, c=FAKE, s=FAKE, t=FAKE,
                a=FAKE, b=FAKE, r=8, ls=2.0, y=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["m"], a["n"], a["k"], a["w"], a["sg"], a["seed"], a["step"], a["nid"], a["eps"], a["c"],
                 a["s"], a["t"], a["a"], a["b"], a["r"], a["ls"], a["y"], a["ws"], a["wsb"], None)

    assert call(m=129) == ERR_SHAPE
    assert call(k=32768) == ERR_SHAPE
    assert call(k=24) == ERR_SHAPE
    assert call(r=257) == ERR_SHAPE
    assert call(sg=-1.0) == ERR_VALUE
    assert call(eps=float("nan")) == ERR_VALUE
    assert call(ls=float("inf")) == ERR_VALUE
    assert call(w=None) == ERR_NULL
    assert call(b=None) == ERR_NULL
    assert call(y=None) == ERR_NULL
    assert call(w=MIS) == ERR_ALIGN
    assert call(t=FAKE + 2) == ERR_ALIGN
    assert call(wsb=ws - 1) == ERR_WORKSPACE
    assert call(ws=None) == ERR_WORKSPACE
    assert call(m=0) == OK and call(n=0) == OK


def test_aqn_rejects_bad_arguments(lib):
    f = lib.fp4rl_aqn_rmsnorm
    assert f(FAKE, 4, 512, FAKE, -1.0, 0, 0, 0, 1e-6, FAKE, None, None) == ERR_VALUE
    assert f(FAKE, 4, 512, FAKE, float("inf"), 0, 0, 0, 1e-6, FAKE, None, None) == ERR_VALUE
    assert f(FAKE, 4, 512, FAKE, 0.01, 0, 0, 0, -1.0, FAKE, None, None) == ERR_VALUE
    assert f(FAKE, 4, 16385, FAKE, 0.01, 0, 0, 0, 1e-6, FAKE, None, None) == ERR_SHAPE
    assert f(FAKE, 4, 512, None, 0.01, 0, 0, 0, 1e-6, FAKE, None, None) == ERR_NULL
    assert f(MIS, 4, 512, FAKE, 0.01, 0, 0, 0, 1e-6, FAKE, None, None) == ERR_ALIGN
    assert f(FAKE, 0, 512, FAKE, 0.01, 0, 0, 0, 1e-6, FAKE, None, None) == OK
    assert lib.fp4rl_philox_words(0, 0, 0, -1, FAKE, None) == ERR_SHAPE
    assert lib.fp4rl_philox_words(0, 0, 0, 4, MIS, None) == ERR_ALIGN


def test_layout_sizes(lib):
    assert lib.fp4rl_nvfp4_codes_bytes(256, 512, 0) == 256 * 256
    assert lib.fp4rl_nvfp4_scales_bytes(256, 512, 0) == 256 * 32
    assert lib.fp4rl_nvfp4_codes_bytes(37, 80, 1) == 3 * 1 * 1024      # 3 row tiles x 1 k chunk
    assert lib.fp4rl_nvfp4_scales_bytes(37, 80, 1) == 3 * 128
    assert lib.fp4rl_nvfp4_codes_bytes(18944, 3584, 1) == 18944 * 3584 // 2
    assert lib.fp4rl_nvfp4_codes_bytes(8, 24, 1) == 0                   # invalid k


def test_aqn_sigma_host_function(lib):
    for k in range(10):
        # the C ABI takes fp32 sigmas: feed the oracle the same fp32 inputs
        want = aqn.sigma_schedule(float(np.float32(1e-2)), float(np.float32(5e-4)), k, 10)
        assert np.float32(lib.fp4rl_aqn_sigma(1e-2, 5e-4, k, 10)) == want
    assert lib.fp4rl_aqn_sigma(0.3, 0.1, 0, 1) == np.float32(0.3)
    assert math.isnan(lib.fp4rl_aqn_sigma(0.3, 0.1, 3, 3))
    assert math.isnan(lib.fp4rl_aqn_sigma(-1.0, 0.1, 0, 3))


def test_valid_call_without_gpu_reports_hip_error(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this checks the no-device path")
    ws = lib.fp4rl_nvfp4_quantize_workspace(8, 32)
    assert lib.fp4rl_nvfp4_quantize(FAKE, 0, 8, 32, 1, FAKE, FAKE, FAKE, FAKE, ws, None) == ERR_HIP
    assert lib.fp4rl_last_error().decode().startswith("hipGetDevice")


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(fr, "LIB_PATH", "/nonexistent/libfp4rl.so")
    monkeypatch.setattr(fr, "_LIB", None)
    with pytest.raises(fr.Fp4rlError):
        fr.load_library()


def test_workspace_check_and_reset_validate_arguments(lib):
    """Argument checks of the hand-off health calls, all decided before any device access."""
    counter_bytes = 4 * (1280 + 64 * 64)
    assert lib.fp4rl_linear_workspace_check(None, 0, None) == OK          # no workspace: no hand-off
    assert lib.fp4rl_linear_workspace_reset(None, 0, None) == OK
    assert lib.fp4rl_linear_workspace_check(FAKE, counter_bytes - 4, None) == ERR_WORKSPACE
    assert lib.fp4rl_linear_workspace_reset(FAKE, 16, None) == ERR_WORKSPACE
    assert lib.fp4rl_linear_workspace_check(FAKE + 4, counter_bytes, None) == ERR_ALIGN
    assert lib.fp4rl_linear_workspace_reset(FAKE + 8, counter_bytes, None) == ERR_ALIGN
    lib.fp4rl_debug_lora_handoff(0, 0)  # the defaults; touches no device


@pytest.mark.parametrize("m,n,k,r,kernel", [
    # decode: one or two tokens, 3..16 tokens, 17..128 tokens
    (1, 18944, 3584, 32, "gemv_kernel<1, 4, 4>"),
    (1, 3584, 18944, 32, "gemv_kernel<1, 16, 4>"),
    (8, 4608, 3584, 32, "skinny_kernel<1, 2, 8>"),
    (32, 18944, 3584, 32, "splitk_kernel<4, 2, 4, 2>"),
    # 97..128 tokens: the mid-batch kernel on wide matrices, with a K split on long K, else split-K
    (128, 27648, 5120, 64, "mid_kernel<1, 2, 4, 2, 3>"),
    (128, 5120, 27648, 64, "mid_kernel<1, 2, 4, 2, 3>"),
    (128, 3584, 18944, 32, "splitk_kernel<4, 2, 4, 2>"),
    # prefill: eight waves where the 512-feature workgroups fill whole rounds of 256, else four
    (8192, 18944, 3584, 32, "prefill_kernel<2, 8>"),
    (8192, 3584, 18944, 32, "prefill_kernel<2, 8>"),
    (8192, 3584, 3584, 32, "prefill_kernel<2, 8>"),
    (8192, 4608, 3584, 32, "prefill_kernel<2, 4>"),
    (8192, 5120, 5120, 32, "prefill_kernel<2, 4>"),
    (2048, 18944, 3584, 32, "prefill_kernel<2, 4>"),
])
def test_kernel_dispatch(lib, m, n, k, r, kernel):
    """The main kernel the library picks for the measured shapes (a host query: no GPU needed)."""
    assert fr.fp4_linear_kernel_name(m, n, k, r) == kernel
