// LoRA up-projection by MFMA for decode-shaped kernels (internal to
// libfp4rl): t = s x A^T (fp32, in K-slices) against the B rows of one 16-row
// output tile, accumulated into the kernel's own MFMA result layout (lane:
// rows 4 g + v of the tile, token li of each 16-token tile).
#pragma once

#include "device.hpp"

namespace fp4rl {

// acc[j] += t[tokens of tile j] . B[rows of tile rt] by MFMA, 32 ranks per
// step: A operand = B row li (ranks 32 q + 8 g .. + 7), B operand = t of
// token 16 j + li split into bf16 hi + lo (two MFMAs: t kept to ~2^-17).
// Rows and tokens past N and M are clamped (never stored), ranks past r zero.
template <int T>
__device__ __forceinline__ void lora_mfma(f32x4 (&acc)[T], const float* __restrict__ t, int tsl,
                                          const uint16_t* __restrict__ b, int r, int M, int N, int rt, int li, int lg) {
  const int64_t tstride = (int64_t)M * r;  // t's K-slices, added in slice order
  const uint16_t* brow = b + (int64_t)min(16 * rt + li, N - 1) * r;
  const bool vec = (r & 7) == 0;
  for (int q0 = 0; q0 < r; q0 += 32) {
    const int q = q0 + 8 * lg;
    uint32_t bw[4];
    if (vec) {
      const uint4 v = q < r ? *reinterpret_cast<const uint4*>(brow + q) : make_uint4(0u, 0u, 0u, 0u);
      bw[0] = v.x; bw[1] = v.y; bw[2] = v.z; bw[3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = q + 2 * e < r ? brow[q + 2 * e] : 0u, hi = q + 2 * e + 1 < r ? brow[q + 2 * e + 1] : 0u;
        bw[e] = lo | (hi << 16);
      }
    }
    const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const float* trow = t + (int64_t)min(16 * j + li, M - 1) * r;
      float tv[8];
      if (vec && q < r) {
        float4 t0 = *reinterpret_cast<const float4*>(trow + q), t1 = *reinterpret_cast<const float4*>(trow + q + 4);
        for (int z = 1; z < tsl; ++z) {
          const float4 u0 = *reinterpret_cast<const float4*>(trow + z * tstride + q);
          const float4 u1 = *reinterpret_cast<const float4*>(trow + z * tstride + q + 4);
          t0.x += u0.x; t0.y += u0.y; t0.z += u0.z; t0.w += u0.w;
          t1.x += u1.x; t1.y += u1.y; t1.z += u1.z; t1.w += u1.w;
        }
        tv[0] = t0.x; tv[1] = t0.y; tv[2] = t0.z; tv[3] = t0.w; tv[4] = t1.x; tv[5] = t1.y; tv[6] = t1.z; tv[7] = t1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = 0.0f;
          if (q + e < r)
            for (int z = 0; z < tsl; ++z) v += trow[z * tstride + q + e];
          tv[e] = v;
        }
      }
      uint4 th, tl;
      split_bf16x8(tv, th, tl);
      acc[j] = mfma16x16x32(a, as_bf16x8(th), acc[j]);
      acc[j] = mfma16x16x32(a, as_bf16x8(tl), acc[j]);
    }
  }
}

}  // namespace fp4rl
