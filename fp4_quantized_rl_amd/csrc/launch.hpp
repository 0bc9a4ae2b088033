// Host-side launchers of the gfx950 kernels (internal to libfp4rl).
// Arguments are already validated by the C ABI layer; each launcher queues
// its kernels on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4rl {

// ---- NVFP4 quantiser --------------------------------------------------
constexpr int kAmaxPartials = 1024;  // workgroups of the amax pass = partial maxima
size_t quantize_workspace_bytes();
hipError_t launch_quantize(const void* w, bool w_bf16, int64_t n, int64_t k, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, uint32_t* partial,
                           hipStream_t stream);

// ---- AQN ----------------------------------------------------------------
constexpr int64_t kAqnMaxD = 16384;  // noise vector lives in LDS (64 KB)
hipError_t launch_aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, const float* w, float sigma,
                              uint64_t seed, uint64_t step, uint32_t norm_id, float eps,
                              uint16_t* y, float* w_noise_out, hipStream_t stream);
hipError_t launch_philox_words(uint64_t seed, uint64_t step, uint32_t norm_id, int64_t n_blocks,
                               uint32_t* out, hipStream_t stream);

// ---- LoRA linear ----------------------------------------------------------
constexpr int64_t kMaxRank = 256;
hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* a, int64_t r,
                            float lora_scale, float* t, hipStream_t stream);
hipError_t launch_fp4_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             const float* t, const uint16_t* b, int64_t r, uint16_t* y,
                             hipStream_t stream);

}  // namespace fp4rl
