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
int64_t nvfp4_codes_bytes(int64_t n, int64_t k, bool tiled);
int64_t nvfp4_scales_bytes(int64_t n, int64_t k, bool tiled);
hipError_t launch_quantize(const void* w, bool w_bf16, int64_t n, int64_t k, bool tiled, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, uint32_t* partial, hipStream_t stream);
hipError_t launch_to_tiled(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, uint8_t* codes_t,
                           uint8_t* scales_t, hipStream_t stream);

// ---- AQN ----------------------------------------------------------------
constexpr int64_t kAqnMaxD = 16384;  // noise vector lives in LDS (64 KB)
hipError_t launch_aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, const float* w, float sigma,
                              uint64_t seed, uint64_t step, uint32_t norm_id, float eps,
                              uint16_t* y, float* w_noise_out, hipStream_t stream);
hipError_t launch_philox_words(uint64_t seed, uint64_t step, uint32_t norm_id, int64_t n_blocks,
                               uint32_t* out, hipStream_t stream);

// ---- LoRA linear ----------------------------------------------------------
constexpr int64_t kMaxRank = 256;
// K-split of the LoRA down-projection: `slices` partial sums [slices][m][r].
int lora_splits(int64_t m, int64_t k, int64_t r);
int lora_slices(int64_t k, int splits);
hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* a, int64_t r, float lora_scale,
                            int splits, float* part, hipStream_t stream);
hipError_t launch_lora_reduce(const float* part, int slices, int64_t count, float* t, hipStream_t stream);
const char* fp4_linear_kernel_name(int64_t m, int64_t n, int64_t k, int64_t r);
// Linear workspaces begin with kLinearCounters counter words (one per output
// tile of a K-split launch; K is split only when there are fewer tiles). They
// must be zero before the first call, and every launch leaves them at zero.
// Its other regions (t slices, K-split partials) follow and never overlap
// the counters, whatever shapes share the workspace.
constexpr int kLinearCounters = 256;
constexpr size_t kLinearCounterBytes = kLinearCounters * sizeof(uint32_t);
// fp32 K-split partial sums of the main kernel (0 when K is not split)
size_t linear_partial_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_fp4_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                             const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                             const float* t, int tks, const uint16_t* b, int64_t r, uint16_t* y, float* part,
                             uint32_t* counters, hipStream_t stream);

}  // namespace fp4rl
