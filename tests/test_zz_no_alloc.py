"""The allocation-free quantiser entry point against the workspace one, through the C ABI (GPU).

fp4rl_nvfp4_quantize_noalloc keeps the amax partials in a library-owned
device array instead of a caller workspace. Two calls in a row, the second on
a smaller matrix (the array keeps the first call's partials), must each give
the same codes, scale bytes and tensor scale, byte for byte, as
fp4rl_nvfp4_quantize with its own workspace, and as the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr
from oracle import nvfp4
from workloads import normal_f32

from gpu_util import device, say

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _quantize_both(lib, dev, w_host, layout):
    n, k = w_host.shape
    w = torch.from_numpy(w_host).to(dev)
    cb, sb = lib.fp4rl_nvfp4_codes_bytes(n, k, layout), lib.fp4rl_nvfp4_scales_bytes(n, k, layout)
    out = []
    for noalloc in (False, True):
        codes = torch.full((cb,), 0xAB, dtype=torch.uint8, device=dev)
        scales = torch.full((sb,), 0xCD, dtype=torch.uint8, device=dev)
        ts = torch.full((1,), -1.0, dtype=torch.float32, device=dev)
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        if noalloc:
            st = lib.fp4rl_nvfp4_quantize_noalloc(_ptr(w), 0, n, k, layout, _ptr(codes), _ptr(scales), _ptr(ts),
                                                  stream)
        else:
            ws = torch.empty(lib.fp4rl_nvfp4_quantize_workspace(n, k), dtype=torch.uint8, device=dev)
            st = lib.fp4rl_nvfp4_quantize(_ptr(w), 0, n, k, layout, _ptr(codes), _ptr(scales), _ptr(ts),
                                          _ptr(ws), ws.numel(), stream)
        assert st == 0, lib.fp4rl_last_error().decode()
        torch.cuda.synchronize()
        out.append((codes.cpu().numpy(), scales.cpu().numpy(), ts.cpu().numpy()))
    return out


@pytest.mark.parametrize("layout", [0, 1])
def test_noalloc_quantize_matches_workspace_entry_point(layout):
    dev = device()
    lib = fr.load_library()
    # a large matrix first (many amax workgroups fill the array), then a smaller ragged one
    for n, k, seed in ((2304, 5120, 11), (37, 272, 12)):
        say(f"nvfp4 quantize noalloc n={n} k={k} layout={layout}")
        w = normal_f32((n, k), 0.02, seed)
        w[n // 2, k // 3] = 0.9  # the tensor amax, placed away from the first workgroups
        (c0, s0, t0), (c1, s1, t1) = _quantize_both(lib, dev, w, layout)
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1), "codes or scales differ"
        assert t0.view(np.uint32)[0] == t1.view(np.uint32)[0], "tensor scale differs"
        codes, scales, st = nvfp4.quantize(w)
        assert np.float32(t1[0]) == st, "tensor scale differs from the oracle"
        if layout == 0:
            assert np.array_equal(c1.reshape(codes.shape), codes) and np.array_equal(s1.reshape(scales.shape), scales)
