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


def nvfp4_to_dev(codes, scales, s_t, dev) -> fr.NVFP4Weight:
    return fr.NVFP4Weight(u8_to_dev(codes, dev), u8_to_dev(scales, dev),
                          torch.tensor([np.float32(s_t)], dtype=torch.float32, device=dev))


def nvfp4_from_dev(wq: fr.NVFP4Weight):
    torch.cuda.synchronize()
    return (wq.codes.cpu().numpy(), wq.scales.cpu().numpy(),
            np.float32(wq.tensor_scale.cpu().numpy()[0]))


def say(msg: str) -> None:
    print(msg, flush=True)
