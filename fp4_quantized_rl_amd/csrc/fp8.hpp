// Host-side launchers of the FP8 (E4M3) rollout weights and their linear
// (internal to libfp4rl); arguments are validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp4rl {

// codes [n][k] E4M3 bytes, scales [n] fp32 (s_n = amax_n / 448)
hipError_t launch_fp8_quantize(const void* w, bool w_bf16, int64_t n, int64_t k, uint8_t* codes, float* scales,
                               hipStream_t stream);

struct Fp8Ws {
  uint8_t* x8 = nullptr;   // [m][k] E4M3 codes of the tokens (W8A8)
  float* xs = nullptr;     // [m] their scales
  uint16_t* xb = nullptr;  // [m][k] the token codes widened to bf16 (W8A8 decode, 17..64 tokens)
  float* ypart = nullptr;  // [S][m][n] partial products of the base (S contraction slices)
  float* tpart = nullptr;  // [St][m][r] K-slices of t = s x A^T
  uint16_t* ts = nullptr;  // [m][2 rp] bf16 hi | lo of t (unsplit launches; rp = r rounded up to 8)
  uint16_t* b2 = nullptr;  // [n][2 rp] bf16 (B | B)
};
// Bytes of the linear's workspace; with `w` and `base`, also its regions.
// a8: W8A8 (tokens quantised to E4M3 with one scale each) instead of W8A16.
size_t fp8_linear_workspace(int64_t m, int64_t n, int64_t k, int64_t r, bool a8, Fp8Ws* w, void* base);
hipError_t launch_fp8_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                             const float* scales, const uint16_t* a, const uint16_t* b, int64_t r, float s, bool a8,
                             uint16_t* y, const Fp8Ws& w, hipStream_t stream);

}  // namespace fp4rl
