"""The decode path under HIP graph capture: every replay equals the eager result bit for bit."""
import numpy as np
import pytest
import torch

import fp4_quantized_rl_amd as fr

from gpu_util import device, say

pytestmark = pytest.mark.gpu


def _inputs(dev, m, n, k, r, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    w = torch.randn((n, k), generator=g, device=dev).mul_(0.02)
    wq = fr.nvfp4_quantize(w)
    x = torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)
    a = torch.randn((r, k), generator=g, device=dev).mul_(0.01).to(torch.bfloat16)
    b = torch.randn((n, r), generator=g, device=dev).mul_(0.01).to(torch.bfloat16)
    return wq, x, a, b


@pytest.mark.parametrize("m,n,k", [(1, 4608, 3584), (8, 4608, 3584), (64, 4608, 3584), (64, 3584, 18944)])
def test_graph_replays_match_eager(m, n, k):
    """The last case splits K over workgroups: its counters must be back at zero after every replay."""
    dev = device()
    r = 32
    wq, x, a, b = _inputs(dev, m, n, k, r, 100 + m + n)
    wn = torch.ones(k, dtype=torch.float32, device=dev)
    ws = fr.linear_workspace(fr.fp4_lora_linear_workspace_bytes(m, n, k, r), dev)
    h = torch.empty_like(x)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

    def path():
        if k <= 16384:  # the norm's width limit; wider inputs go to the linear as they are
            fr.aqn_rmsnorm(x, wn, 1e-2, 7, 3, 0, 1e-6, out=h)
        else:
            h.copy_(x)
        fr.fp4_lora_linear(h, wq, a, b, 2.0, out=y, workspace=ws)

    path()
    torch.cuda.synchronize()
    h_ref, y_ref = h.clone(), y.clone()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        path()
    other_wq, other_x, other_a, other_b = _inputs(dev, 5, 256, 512, 8, 7)
    for i in range(4):
        h.zero_()
        y.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref), f"replay {i}: norm output differs"
        assert torch.equal(y, y_ref), f"replay {i}: linear output differs"
        fr.fp4_lora_linear(other_x, other_wq, other_a, other_b, 2.0)  # unrelated eager work in between
        torch.cuda.synchronize()
    say(f"  M={m} {n}x{k}: 4 replays identical to eager")


@pytest.mark.parametrize("layout,dtype", [("tiled", torch.float32), ("row_major", torch.bfloat16)])
def test_quantizer_graph_replays_match_eager(layout, dtype):
    """The quantiser (both passes, with the rounding record) captured in a graph, ragged in n and k:
    every replay writes the eager codes, scale bytes, tensor scale and record (no memset nodes)."""
    dev = device()
    n, k = 300, 1296
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    w = torch.randn((n, k), generator=g, device=dev).mul_(0.02).to(dtype)
    out = fr.nvfp4_empty(n, k, layout, dev)
    ru = torch.empty((n, k // 8), dtype=torch.uint8, device=dev)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    fr.nvfp4_quantize(w, layout=layout, out=out, workspace=ws, round_up=ru)
    torch.cuda.synchronize()
    ref = [out.codes.clone(), out.scales.clone(), out.tensor_scale.clone(), ru.clone()]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        fr.nvfp4_quantize(w, layout=layout, out=out, workspace=ws, round_up=ru)
    other = torch.randn((64, 256), generator=g, device=dev)
    for i in range(4):
        for t in (out.codes, out.scales, out.tensor_scale, ru):
            t.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = [out.codes, out.scales, out.tensor_scale, ru]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {i} differs from eager"
        fr.nvfp4_quantize(other, layout="tiled")  # unrelated eager work in between (its own workspace)
        torch.cuda.synchronize()
    say(f"  quantiser {layout} {dtype}: 4 replays identical to eager")


def _replays_match(dev, path, outs, other):
    path()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        path()
    for i in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), f"replay {i}: output differs from eager"
        other()  # unrelated eager work in between
        torch.cuda.synchronize()


@pytest.mark.parametrize("m", [1, 8, 64, 256])
def test_fp8_linear_graph_replays(m):
    """Decode (partials + finishing pass) and the one-launch prefill path under capture."""
    dev = device()
    n, k, r = 4608, 3584, 32
    _, x, a, b = _inputs(dev, m, n, k, r, 300 + m)
    w8 = fr.fp8_quantize(torch.randn((n, k), device=dev).mul_(0.02))
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(256, fr.fp8_lora_linear_workspace_bytes(m, n, k, r)), dtype=torch.uint8, device=dev)
    other = (lambda: fr.fp8_lora_linear(x[:1], w8, a, b, 2.0))
    _replays_match(dev, lambda: fr.fp8_lora_linear(x, w8, a, b, 2.0, out=y, workspace=ws), [y], other)
    say(f"  FP8 M={m}: 4 replays identical to eager")


@pytest.mark.parametrize("m", [4, 40])
def test_gate_up_graph_replays(m):
    dev = device()
    n, k, r = 4608, 3584, 16
    wq, x, a, b = _inputs(dev, m, n, k, r, 400 + m)
    wu, _, a2, b2 = _inputs(dev, m, n, k, r, 500 + m)
    h = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    # counter words zero before the first call, as the workspace contract asks
    ws = torch.zeros(max(256, fr.load_library().fp4rl_fp4_gate_up_silu_workspace(m, n, k, r)), dtype=torch.uint8,
                     device=dev)
    other = (lambda: fr.fp4_gate_up_silu(x[:1], wq, wu, (a, b), (a2, b2), 2.0))
    _replays_match(dev, lambda: fr.fp4_gate_up_silu(x, wq, wu, (a, b), (a2, b2), 2.0, out=h, workspace=ws), [h],
                   other)
    say(f"  gate/up M={m}: 4 replays identical to eager")


def test_backward_graph_replays():
    dev = device()
    m, n, k, r = 200, 1024, 768, 16
    wq, x, a, b = _inputs(dev, m, n, k, r, 600)
    dy = torch.randn((m, n), device=dev).mul_(0.05).to(torch.bfloat16)
    ws = torch.empty(fr.fp4_lora_linear_backward_workspace_bytes(m, n, k, r), dtype=torch.uint8, device=dev)
    outs = {}

    def path():
        outs["r"] = fr.fp4_lora_linear_backward(dy, x, wq, a, b, 2.0, workspace=ws)

    # the call allocates its outputs: the tensors it returns while being
    # captured (from the graph's memory pool) are the ones every replay writes
    path()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs["r"]]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        path()
    got = outs["r"]
    for i in range(4):
        for t in got:
            t.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for t, rf in zip(got, ref):
            assert torch.equal(t, rf), f"replay {i}: backward output differs from eager"
        fr.fp4_lora_linear_backward(dy[:8], x[:8], wq, a, b, 2.0)
        torch.cuda.synchronize()
    say("  backward: 4 replays identical to eager")
