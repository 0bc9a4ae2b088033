// Host-side launcher of the LoRA backward (internal to libfp4rl); arguments
// are validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4rl {

// Workspace regions of the backward (see backward_workspace): the transposed
// dequantised weight, the transposed adapters and activations, t and h split
// into bf16 hi | lo, and fp32 partial products.
struct BackwardWs {
  uint16_t* wt = nullptr;   // [k][n] bf16, g S_b (dX only)
  uint16_t* bt = nullptr;   // [r][n] bf16
  uint16_t* at2 = nullptr;  // [k][2 rp] bf16, (A^T | A^T), rp = r rounded up to 8 (dX only)
  uint16_t* dyt = nullptr;  // [n][mp] bf16, dY transposed (mp = m rounded up to 8; tokens past m zero)
  uint16_t* xt = nullptr;   // [k][mp] bf16, x transposed
  uint16_t* hs = nullptr;   // [m][2 rp] bf16 hi | lo of h = s dY B (dX only)
  uint16_t* hst = nullptr;  // [2 rp][mp] bf16, hi | lo of h transposed
  uint16_t* tst = nullptr;  // [2 rp][mp] bf16, hi | lo of t = s x A^T transposed
  float* part = nullptr;    // fp32 partial products of the contraction-split launches
};
// Bytes of the backward workspace; with `w` and `base`, also its regions.
size_t backward_workspace(int64_t m, int64_t n, int64_t k, int64_t r, bool want_dx, BackwardWs* w, void* base);
hipError_t launch_lora_backward(const uint16_t* dy, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                const uint16_t* a, const uint16_t* b, int64_t r, float s, uint16_t* dx, float* da,
                                float* db, const BackwardWs& w, hipStream_t stream);
// Sets `words` 32-bit words at p to zero (a kernel, not a memset).
hipError_t launch_zero_words(void* p, int64_t words, hipStream_t stream);

}  // namespace fp4rl
