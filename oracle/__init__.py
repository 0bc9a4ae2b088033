"""CPU oracle for the NVFP4 + LoRA + AQN hot path — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy (float64) implementations of what the
rollout hot path computes:

* ``nvfp4``  – the NVFP4 block quantiser (16-element blocks, one E4M3 scale
  per block, one FP32 tensor scale, values on the E2M1 grid), its exact
  dequantisation and the per-value rounding record (rounded up or down);
* ``linear`` – y = x deq(Wq)^T + s (x A^T) B^T, the W4A16 linear with the
  LoRA update;
* ``lora_backward`` – dX, dA and dB of that linear (the base stays frozen);
* ``fp8``    – the FP8 (E4M3, per-row scale) rollout weights and their W8A16 linear;
* ``gate_up`` – gate and up projections of one input with the SiLU-gated product;
* ``aqn``    – the Adaptive Quantization Noise RMSNorm: the exponential sigma
  schedule, Philox4x32-10 + Box-Muller noise, and the noisy-weight RMSNorm;
* ``numerics`` – bf16 round-to-nearest-even and the rel-L2 metric.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product library
(``fp4_quantized_rl_amd``) never imports, links or calls anything here, and the
two share no code: the only common module is ``workloads`` (seeded inputs).

Parity status of each function is stated in its docstring; every function
here is pinned by a ``-m "not gpu"`` test against something other than
itself (closed forms, brute force, torch CPU casts, torch's Philox header),
except where a docstring says "parity unpinned".
"""
from . import numerics, nvfp4, linear, lora_backward, fp8, gate_up, aqn  # noqa: F401
