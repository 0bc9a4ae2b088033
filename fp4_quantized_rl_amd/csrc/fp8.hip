// FP8 (OCP E4M3) rollout weights and their W8A16 / W8A8 linear with LoRA
// (gfx950).
//
// Low-precision rollout engines commonly run the policy in FP8 while the
// trainer keeps BF16 (gist.science summary of adaptive importance sampling
// for quantized RL, "Problem definition"); FP8 halves the rollout model's
// memory ("Experimental results"). Format: one E4M3 byte per weight, one
// fp32 scale per output row, s_n = amax_n / 448; the code of w is the
// nearest E4M3 value to the fp32 quotient w / s_n (ties to even, saturating
// at 448, no -0). The linear is
//   y = bf16(sum_k x[m,k] e4m3(code[n,k]) s_n + s (x A^T)[m] . B[n]).
//
// Kernels:
//   fp8_quantize_kernel: one workgroup per row: the row's amax (exact max of
//     |w| bit patterns), s_n, then the codes, 16 bytes per store.
//   nt_gemm_kernel<false, 1, kNtR8>: x (bf16) against the E4M3 rows, converted
//     to bf16 exactly on the way into LDS (v_cvt_pk_f32_fp8), fp32
//     accumulation scaled per row by s_n; the contraction is split over
//     workgroups when there are few output tiles (decode), partials fp32.
//   Decode, 17..64 tokens: the NVFP4 linear's split-K kernel in its E4M3
//     mode (activations staged through LDS); without a K split it stores y
//     itself (row scales, t B^T by MFMA), else fp32 partials. W8A8 gives it
//     the token codes widened to bf16 (exact; written by the token
//     quantiser) and multiplies by the token scales: the same exact E4M3
//     products, accumulated in fp32, as on the FP8 matrix cores.
//   Decode up to 16 tokens: fp8_decode_kernel / e4m3_decode_kernel, fp32
//     partials per K-slice.
//   t = s x A^T in K-slices by the NVFP4 linear's LoRA down-projection
//   kernel; the finishing kernels add the slices in order. With enough output tiles (prefill) the linear writes
//   bf16 y in one launch, the LoRA term accumulated as a second contraction
//   segment (t as bf16 hi | lo against B twice: lora_operands_kernel);
//   split (decode), fp8_finish_kernel makes y = bf16(sum of slices + t . B[n]):
//   a workgroup per 256 features x 2 tokens, t's K-slices summed once into
//   LDS (it was once per output and rank: 38.5 -> 14.7 us for the 7B gate at
//   64 tokens).
// W8A8: the tokens are quantised like weight rows (one E4M3 scale per token,
//   fp8_quantize_kernel into the workspace), the base product runs on the
//   FP8 matrix cores with both operands as bytes (e4m3_decode_kernel,
//   nt_gemm_kernel<., 1, kNtE4M3>), scaled by s_n xs[m]; the LoRA term still
//   reads the bf16 tokens.
#include <algorithm>

#include "device.hpp"
#include "fp8.hpp"
#include "gemm_nt.hpp"
#include "launch.hpp"

namespace fp4rl {
namespace {

// Nearest finite E4M3 magnitude byte to a non-negative fp32 value, ties to
// even (round to 3 mantissa bits; subnormals are multiples of 2^-9).
__device__ __forceinline__ uint32_t e4m3_rne(float a) {
  if (!(a < 448.0f)) return 0x7Eu;  // saturate (a >= 448, or rounding up past 448 below)
  if (a < 0x1p-6f) return (uint32_t)__builtin_rintf(a * 512.0f);  // subnormal: m 2^-9, m = 8 is 2^-6 (byte 0x08)
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // round the 23-bit mantissa to 3 bits, ties to even
  const uint32_t e = (u >> 23) - 120u, m = (u >> 20) & 7u;  // E4M3 exponent field: unbiased + 7
  return min((e << 3) | m, 0x7Eu);
}

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* w, int64_t i) {
  if constexpr (BF16) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(w) + i);
    return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(w) + i);
  }
}

// wide (optional): the codes' values as bf16 (exact: 4 significant bits)
template <bool BF16>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const void* __restrict__ w, int K,
                                                           uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                           uint16_t* __restrict__ wide = nullptr) {
  __shared__ uint32_t red[4];
  const int64_t row = blockIdx.x;
  const int64_t base = row * K;
  uint32_t mx = 0;
  for (int k = 4 * threadIdx.x; k < K; k += 1024) {
    const float4 v = load4<BF16>(w, base + k);
    mx = max(mx, max(max(__float_as_uint(v.x) & 0x7FFFFFFFu, __float_as_uint(v.y) & 0x7FFFFFFFu),
                     max(__float_as_uint(v.z) & 0x7FFFFFFFu, __float_as_uint(v.w) & 0x7FFFFFFFu)));
  }
  mx = wave_max_u32(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = max(max(red[0], red[1]), max(red[2], red[3]));
  const float s = __uint_as_float(mx) / 448.0f;  // correctly rounded division
  if (threadIdx.x == 0) scales[row] = s;
  // 16 elements per thread and step: four float4 loads, one 16-byte store
  for (int k = 16 * threadIdx.x; k < K; k += 4096) {
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float4 v = load4<BF16>(w, base + k + 4 * d);
      const float f[4] = {v.x, v.y, v.z, v.w};
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float q = s > 0.0f ? f[e] / s : 0.0f;
        uint32_t c = e4m3_rne(fabsf(q));
        if (q < 0.0f && c != 0u) c |= 0x80u;
        word |= c << (8 * e);
      }
      o[d] = word;
    }
    *reinterpret_cast<uint4*>(codes + base + k) = make_uint4(o[0], o[1], o[2], o[3]);
    if (wide != nullptr) {
      uint32_t h[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(o[d], false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(o[d], true);
        h[2 * d] = pack_hi16(lo.x, lo.y);
        h[2 * d + 1] = pack_hi16(hi.x, hi.y);
      }
      *reinterpret_cast<uint4*>(wide + base + k) = make_uint4(h[0], h[1], h[2], h[3]);
      *reinterpret_cast<uint4*>(wide + base + k + 8) = make_uint4(h[4], h[5], h[6], h[7]);
    }
  }
}

// y[m][n] = bf16(sum_s part[s][m][n] + sum_j t[m][j] B[n][j]), t the sum of
// its K-slices tpart[q][m][j]; slices, K-slices and ranks in order. A
// workgroup takes 256 features x kFinTok tokens: its tokens' t rows (K-slices
// summed) are staged in LDS once, and each thread, one feature, reads its B
// row 8 ranks at a time and accumulates the rank products of every token.
constexpr int kFinTok = 2;
template <int FT>
__global__ __launch_bounds__(256) void fp8_finish_kernel(const float* __restrict__ part, int slices, int M, int N,
                                                         const float* __restrict__ tpart, int tsl,
                                                         const uint16_t* __restrict__ b, int r,
                                                         uint16_t* __restrict__ y) {
  extern __shared__ float tsh[];  // [FT][r]
  const int64_t count = (int64_t)M * N, tstride = (int64_t)M * r;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const uint16_t* bn = b + (int64_t)min(n, N - 1) * r;
  // up to 64 ranks of the B row (r % 8 == 0) are loaded once, all at once,
  // before any rank product; other r read it 8 ranks at a time
  constexpr int kBRegs = 8;
  const bool breg = r <= 8 * kBRegs && (r & 7) == 0;
  uint4 bw[kBRegs];
  if (breg) {
#pragma unroll
    for (int q = 0; q < kBRegs; ++q) bw[q] = 8 * q < r ? *reinterpret_cast<const uint4*>(bn + 8 * q) : make_uint4(0, 0, 0, 0);
  }
  for (int m0 = blockIdx.y * FT; m0 < M; m0 += gridDim.y * FT) {  // uniform across the workgroup
    const int mt = min(FT, M - m0);
    // the partial sums first: their loads are in flight during the t staging
    float v[FT];
#pragma unroll
    for (int mm = 0; mm < FT; ++mm) {
      v[mm] = 0.0f;
      if (n < N && mm < mt) {
        const int64_t i = (int64_t)(m0 + mm) * N + n;
        for (int s = 0; s < slices; ++s) v[mm] += part[(int64_t)s * count + i];
      }
    }
    __syncthreads();  // the previous token block's t is no longer read
    for (int e = threadIdx.x; e < mt * r; e += 256) {
      const int mm = e / r, j = e - mm * r;
      const float* tp = tpart + (int64_t)(m0 + mm) * r + j;
      float tj = tp[0];
      for (int q = 1; q < tsl; ++q) tj += tp[q * tstride];
      tsh[mm * r + j] = tj;
    }
    __syncthreads();
    float l[FT];
#pragma unroll
    for (int mm = 0; mm < FT; ++mm) l[mm] = 0.0f;
    if (breg) {
#pragma unroll
      for (int q = 0; q < kBRegs; ++q) {
        if (8 * q >= r) break;  // uniform
        const float bv[8] = {bf16_lo(bw[q].x), bf16_hi(bw[q].x), bf16_lo(bw[q].y), bf16_hi(bw[q].y),
                             bf16_lo(bw[q].z), bf16_hi(bw[q].z), bf16_lo(bw[q].w), bf16_hi(bw[q].w)};
#pragma unroll
        for (int mm = 0; mm < FT; ++mm)
          if (mm < mt) {
#pragma unroll
            for (int e = 0; e < 8; ++e) l[mm] = fmaf(tsh[mm * r + 8 * q + e], bv[e], l[mm]);
          }
      }
    } else {
      for (int j0 = 0; j0 < r; j0 += 8) {
        float bv[8];
        if ((r & 7) == 0) {  // the B row is 16-byte aligned
          const uint4 w = *reinterpret_cast<const uint4*>(bn + j0);
          bv[0] = bf16_lo(w.x); bv[1] = bf16_hi(w.x); bv[2] = bf16_lo(w.y); bv[3] = bf16_hi(w.y);
          bv[4] = bf16_lo(w.z); bv[5] = bf16_hi(w.z); bv[6] = bf16_lo(w.w); bv[7] = bf16_hi(w.w);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) bv[e] = j0 + e < r ? bf16_lo(bn[j0 + e]) : 0.0f;
        }
        const int je = min(8, r - j0);
#pragma unroll
        for (int mm = 0; mm < FT; ++mm)
          if (mm < mt) {
            for (int e = 0; e < je; ++e) l[mm] = fmaf(tsh[mm * r + j0 + e], bv[e], l[mm]);
          }
      }
    }
    if (n < N) {
#pragma unroll
      for (int mm = 0; mm < FT; ++mm)
        if (mm < mt) y[(int64_t)(m0 + mm) * N + n] = (uint16_t)f32_to_bf16(v[mm] + l[mm]);
    }
  }
}

// ts[m][0..2rp) = bf16 hi | lo of t[m][0..r) (its K-slices summed in order; zero past r); b2[n][0..2rp) =
// (B[n] | B[n]) (zero past r): the LoRA term as a second contraction segment
__global__ __launch_bounds__(256) void lora_operands_kernel(const float* __restrict__ t, int tsl,
                                                            const uint16_t* __restrict__ b, int M, int N, int r, int rp,
                                                            uint16_t* __restrict__ ts, uint16_t* __restrict__ b2) {
  const int64_t nt = (int64_t)M * rp, count = nt + (int64_t)N * rp;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    if (i < nt) {
      const int m = (int)(i / rp), j = (int)(i - (int64_t)m * rp);
      float v = 0.0f;
      if (j < r)
        for (int q = 0; q < tsl; ++q) v += t[(int64_t)q * M * r + (int64_t)m * r + j];
      const uint32_t hb = f32_to_bf16(v);
      ts[(int64_t)m * 2 * rp + j] = (uint16_t)hb;
      ts[(int64_t)m * 2 * rp + rp + j] = (uint16_t)f32_to_bf16(v - __uint_as_float(hb << 16));
    } else {
      const int64_t e = i - nt;
      const int n = (int)(e / rp), j = (int)(e - (int64_t)n * rp);
      const uint16_t v = j < r ? b[(int64_t)n * r + j] : (uint16_t)0;
      b2[(int64_t)n * 2 * rp + j] = v;
      b2[(int64_t)n * 2 * rp + rp + j] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode (W8A16 up to 16 tokens): a workgroup takes 64 weight rows (four 16-row MFMA
// tiles) and one K-slice; its four waves take the slice's 64-k chunks in
// turn (adjacent chunks of the same rows at once), two chunks in flight per
// wave. A lane loads 16 E4M3 bytes per weight tile and chunk straight into
// registers (row li, k = 16 g .. + 15 of the chunk) and converts them
// exactly to bf16; its token fragments (token li, the same 16 k) come from
// x through the cache. The MFMA's k order is permuted the same way on both
// operands (slot (step s, group g, e) holds k = 16 g + 8 s + e), so the sum
// is unchanged. The waves' sums are added in wave order through LDS, scaled
// by s_n and written as fp32 partials [slice][M][N]; fp8_finish_kernel adds
// the slices and the LoRA term.
// ---------------------------------------------------------------------------
constexpr int kDecRows = 64;

template <int T>
__global__ __launch_bounds__(256) void fp8_decode_kernel(const uint16_t* __restrict__ x, int M, int N, int K,
                                                         const uint8_t* __restrict__ codes,
                                                         const float* __restrict__ scales, int slice,
                                                         float* __restrict__ part) {
  __shared__ f32x4 red[3][4 * T][64];
  const int k0 = blockIdx.y * slice, klen = min(slice, K - k0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kDecRows;
  const uint8_t* wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wrow[i] = codes + (int64_t)min(n0 + 16 * i + li, N - 1) * K + k0 + 16 * lg;
  const uint16_t* xrow[T];  // tokens past M are clamped (their columns are never stored)
#pragma unroll
  for (int j = 0; j < T; ++j) xrow[j] = x + (int64_t)min(16 * j + li, M - 1) * K + k0 + 16 * lg;
  f32x4 acc[4][T];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < T; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = (klen + 63) / 64;
  for (int c0 = wave; c0 < nch; c0 += 8) {
    uint4 wv[2][4], xv[2][T][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ch = c0 + 4 * u;
      const bool in = ch < nch && 64 * ch + 16 * lg < klen;  // klen % 16 == 0: all 16 values in or out
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[u][i] = in ? ld_nt16(wrow[i] + 64 * ch) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int j = 0; j < T; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          xv[u][j][h] = in ? *reinterpret_cast<const uint4*>(xrow[j] + 64 * ch + 8 * h) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 a[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w4[4] = {wv[u][i].x, wv[u][i].y, wv[u][i].z, wv[u][i].w};
        uint32_t o[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w4[d], false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(w4[d], true);
          o[2 * d] = pack_hi16(lo.x, lo.y);
          o[2 * d + 1] = pack_hi16(hi.x, hi.y);
        }
        a[0][i] = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
        a[1][i] = __builtin_bit_cast(bf16x8, make_uint4(o[4], o[5], o[6], o[7]));
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int j = 0; j < T; ++j) {
          const bf16x8 b = as_bf16x8(xv[u][j][st]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i][j] = mfma16x16x32(a[st][i], b, acc[i][j]);
        }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < T; ++j) red[wave - 1][i * T + j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave > 0) return;
  // lane holds rows n0 + 16 i + 4 g + v of token 16 j + li
  float* out = part + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + 16 * i + 4 * lg;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const f32x4 v = ((acc[i][j] + red[0][i * T + j][lane]) + red[1][i * T + j][lane]) + red[2][i * T + j][lane];
      const int m = 16 * j + li;
      if (m >= M) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) out[(int64_t)m * N + n + e] = v[e] * scales[n + e];
    }
  }
}

// W8A8 decode: the same work split, with the tokens' E4M3 bytes x8 [M][K]
// and per-token scales xs [M]. A chunk is 128 k; a lane loads bytes
// 16 g .. + 15 and 64 + 16 g .. + 15 of its weight row's and token's chunk
// straight into the FP8 MFMA's operand registers (no conversion; the same
// slots on both operands). Partials are scaled by s_n xs[m].
template <int T>
__global__ __launch_bounds__(256) void e4m3_decode_kernel(const uint8_t* __restrict__ x8, const float* __restrict__ xs,
                                                          int M, int N, int K, const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scales, int slice,
                                                          float* __restrict__ part) {
  __shared__ f32x4 red[3][4 * T][64];
  const int k0 = blockIdx.y * slice, klen = min(slice, K - k0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kDecRows;
  const uint8_t* wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wrow[i] = codes + (int64_t)min(n0 + 16 * i + li, N - 1) * K + k0 + 16 * lg;
  const uint8_t* xrow[T];  // tokens past M are clamped (their columns are never stored)
#pragma unroll
  for (int j = 0; j < T; ++j) xrow[j] = x8 + (int64_t)min(16 * j + li, M - 1) * K + k0 + 16 * lg;
  f32x4 acc[4][T];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < T; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nch = (klen + 127) / 128;
  for (int c0 = wave; c0 < nch; c0 += 8) {
    uint4 wv[2][4][2], xv[2][T][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ch = c0 + 4 * u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int off = 128 * ch + 64 * h;
        const bool in = ch < nch && off + 16 * lg < klen;  // klen % 16 == 0: all 16 bytes in or out
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[u][i][h] = in ? ld_nt16(wrow[i] + off) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < T; ++j)
          xv[u][j][h] = in ? *reinterpret_cast<const uint4*>(xrow[j] + off) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < T; ++j) {
        const i32x8 b = as_i32x8(xv[u][j][0], xv[u][j][1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma16x16x128_e4m3(as_i32x8(wv[u][i][0], wv[u][i][1]), b, acc[i][j]);
      }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < T; ++j) red[wave - 1][i * T + j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave > 0) return;
  // lane holds rows n0 + 16 i + 4 g + v of token 16 j + li
  float* out = part + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int j = 0; j < T; ++j) {
    const int m = 16 * j + li;
    if (m >= M) continue;
    const float sx = xs[m];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 16 * i + 4 * lg;
      const f32x4 v = ((acc[i][j] + red[0][i * T + j][lane]) + red[1][i * T + j][lane]) + red[2][i * T + j][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) out[(int64_t)m * N + n + e] = v[e] * (scales[n + e] * sx);
    }
  }
}

// K-slices of the decode kernels (up to 16 tokens: one token tile): about
// 512 workgroups (64-row groups x slices), each slice a multiple of the
// chunk (64, or 128 for E4M3 tokens) and at least 256 long.
struct DecSplit {
  int slice = 0, slices = 0;
};
DecSplit dec_split(int64_t m, int64_t n, int64_t k, int chunk) {
  (void)m;
  DecSplit d;
  const int64_t groups = (n + kDecRows - 1) / kDecRows;
  int64_t want = (512 + groups - 1) / groups;
  want = std::max<int64_t>(1, std::min<int64_t>(want, k / 256));
  const int64_t len = ((k + want - 1) / want + chunk - 1) / chunk * chunk;
  d.slice = (int)len;
  d.slices = (int)((k + len - 1) / len);
  return d;
}

unsigned flat_grid8(int64_t count) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((count + 255) / 256, 8192));
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

dim3 finish_grid(int64_t m, int64_t n, int ft = kFinTok) {
  return dim3((unsigned)((n + 255) / 256), (unsigned)std::min<int64_t>((m + ft - 1) / ft, 4096));
}
size_t finish_lds(int64_t r, int ft = kFinTok) { return (size_t)ft * (size_t)r * sizeof(float); }

}  // namespace

constexpr int kPartFinTok = 2;  // tokens per workgroup of the NVFP4 K-split finish

hipError_t launch_partials_finish(const float* part, int slices, int64_t m, int64_t n, const float* t, int tks,
                                  const uint16_t* b, int64_t r, uint16_t* y, hipStream_t stream) {
  hipLaunchKernelGGL(fp8_finish_kernel<kPartFinTok>, finish_grid(m, n, kPartFinTok), dim3(256),
                     finish_lds(r, kPartFinTok), stream, part, slices, (int)m, (int)n, t, tks, b, (int)r, y);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void* w, bool w_bf16, int64_t n, int64_t k, uint8_t* codes, float* scales,
                               hipStream_t st) {
  if (w_bf16)
    hipLaunchKernelGGL(fp8_quantize_kernel<true>, dim3((unsigned)n), dim3(256), 0, st, w, (int)k, codes, scales);
  else
    hipLaunchKernelGGL(fp8_quantize_kernel<false>, dim3((unsigned)n), dim3(256), 0, st, w, (int)k, codes, scales);
  return hipGetLastError();
}

// Workspace: W8A8 token codes x8 [m][k] and scales xs [m]; y partials
// [S][m][n] fp32 for decode or a split contraction; with adapters the
// K-slices of t [St][m][r] fp32 and, unsplit, the bf16 LoRA segment operands
// ts [m][2 rp], b2 [n][2 rp].
size_t fp8_linear_workspace(int64_t m, int64_t n, int64_t k, int64_t r, bool a8, Fp8Ws* w, void* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al256(bytes);
    return base ? reinterpret_cast<float*>(static_cast<uint8_t*>(base) + o) : nullptr;
  };
  Fp8Ws v{};
  if (a8) {
    v.x8 = reinterpret_cast<uint8_t*>(take((size_t)m * k));
    v.xs = take((size_t)m * 4);
    if (m > 16 && m <= 64) v.xb = reinterpret_cast<uint16_t*>(take((size_t)m * k * 2));
  }
  // decode (m <= 64) always writes partials; otherwise only a split contraction does
  const bool dec = m <= 64;
  const int chunk = a8 ? 128 : kGC;
  const int sl = dec ? (m <= 16 ? dec_split(m, n, k, chunk).slices : fp8_splitk_slices(m, n, k))
                     : nt_slices(nt_tiles(m, n), k, chunk);
  const bool parts = dec || sl > 1;
  const int64_t rp = (r + 7) / 8 * 8;
  if (parts) v.ypart = take((size_t)sl * m * n * 4);
  if (r > 0) {
    v.tpart = take((size_t)lora_slices(k, lora_splits(m, k, r)) * m * r * 4);
    if (!parts) {
      v.ts = reinterpret_cast<uint16_t*>(take((size_t)m * 2 * rp * 2));
      v.b2 = reinterpret_cast<uint16_t*>(take((size_t)n * 2 * rp * 2));
    }
  }
  if (w) *w = v;
  return off;
}

namespace {

template <int T>
void launch_decode(bool a8, dim3 grid, const uint16_t* x, const Fp8Ws& w, int64_t m, int64_t n, int64_t k,
                   const uint8_t* codes, const float* scales, int slice, hipStream_t st) {
  if (a8)
    hipLaunchKernelGGL(e4m3_decode_kernel<T>, grid, dim3(256), 0, st, w.x8, w.xs, (int)m, (int)n, (int)k, codes, scales,
                       slice, w.ypart);
  else
    hipLaunchKernelGGL(fp8_decode_kernel<T>, grid, dim3(256), 0, st, x, (int)m, (int)n, (int)k, codes, scales, slice,
                       w.ypart);
}

template <int MODE>
void launch_gemm(bool split, int64_t tiles, int sl, const Seg& sw, const Seg& lora, int64_t m, int64_t n,
                 const float* scales, uint16_t* y, float* ypart, hipStream_t st) {
  if (!split)
    hipLaunchKernelGGL((nt_gemm_kernel<true, 1, MODE>), dim3((unsigned)tiles), dim3(256), 0, st, sw, lora, (int)m,
                       (int)n, nullptr, 1.0f, scales, y, nullptr);
  else
    hipLaunchKernelGGL((nt_gemm_kernel<false, 1, MODE>), dim3((unsigned)tiles, (unsigned)sl), dim3(256), 0, st, sw,
                       Seg{}, (int)m, (int)n, nullptr, 1.0f, scales, nullptr, ypart);
}

}  // namespace

hipError_t launch_fp8_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                             const float* scales, const uint16_t* a, const uint16_t* b, int64_t r, float s, bool a8,
                             uint16_t* y, const Fp8Ws& w, hipStream_t st) {
  if (a8) {  // the tokens' E4M3 codes and scales: the weight quantiser, one workgroup per token
    hipLaunchKernelGGL(fp8_quantize_kernel<true>, dim3((unsigned)m), dim3(256), 0, st, x, (int)k, w.x8, w.xs, w.xb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int tsl = 0;
  if (r > 0) {  // t = s x A^T in K-slices from the bf16 tokens (the NVFP4 linear's LoRA down-projection kernel)
    const int splits = lora_splits(m, k, r);
    tsl = lora_slices(k, splits);
    const hipError_t e = launch_lora_down(x, m, k, a, r, s, splits, w.tpart, st);
    if (e != hipSuccess) return e;
  }
  const int chunk = a8 ? 128 : kGC;
  if (m > 16 && m <= 64) {  // decode: the split-K kernel's E4M3 mode (+ the finishing launch for a K split);
                            // W8A8 feeds it the token codes widened to bf16 and their scales
    const hipError_t e = launch_fp8_splitk(a8 ? w.xb : x, m, n, k, codes, scales, w.tpart, tsl, r > 0 ? b : nullptr,
                                           r, y, w.ypart, a8 ? w.xs : nullptr, st);
    if (e != hipSuccess) return e;
    const int sl = fp8_splitk_slices(m, n, k);
    if (sl > 1)
      hipLaunchKernelGGL(fp8_finish_kernel<kFinTok>, finish_grid(m, n), dim3(256), finish_lds(r), st, w.ypart, sl, (int)m,
                         (int)n, w.tpart, tsl, r > 0 ? b : nullptr, (int)r, y);
    return hipGetLastError();
  }
  if (m <= 16) {  // one token tile
    const DecSplit d = dec_split(m, n, k, chunk);
    const dim3 grid((unsigned)((n + kDecRows - 1) / kDecRows), (unsigned)d.slices);
    launch_decode<1>(a8, grid, x, w, m, n, k, codes, scales, d.slice, st);
    hipLaunchKernelGGL(fp8_finish_kernel<kFinTok>, finish_grid(m, n), dim3(256), finish_lds(r), st, w.ypart, d.slices, (int)m,
                       (int)n, w.tpart, tsl, r > 0 ? b : nullptr, (int)r, y);
    return hipGetLastError();
  }
  const int64_t tiles = nt_tiles(m, n);
  const Seg sw = a8 ? Seg{w.x8, codes, (int)k, (int)k, nt_slice_len(tiles, k, chunk), w.xs}
                    : Seg{x, codes, (int)k, (int)k, nt_slice_len(tiles, k, chunk)};
  const int sl = nt_slices(tiles, k, chunk);
  Seg lora{};
  if (sl == 1 && r > 0) {
    // enough output tiles (prefill): bf16 out in one launch, the LoRA term as
    // a second segment (t split into bf16 hi | lo against B twice)
    const int64_t rp = (r + 7) / 8 * 8;
    hipLaunchKernelGGL(lora_operands_kernel, dim3(flat_grid8((m + n) * rp)), dim3(256), 0, st, w.tpart, tsl, b, (int)m,
                       (int)n, (int)r, (int)rp, w.ts, w.b2);
    lora = Seg{w.ts, w.b2, (int)(2 * rp), (int)(2 * rp), (int)(2 * rp)};
  }
  if (a8)
    launch_gemm<kNtE4M3>(sl > 1, tiles, sl, sw, lora, m, n, scales, y, w.ypart, st);
  else
    launch_gemm<kNtR8>(sl > 1, tiles, sl, sw, lora, m, n, scales, y, w.ypart, st);
  if (sl > 1)
    hipLaunchKernelGGL(fp8_finish_kernel<kFinTok>, finish_grid(m, n), dim3(256), finish_lds(r), st, w.ypart, sl, (int)m, (int)n,
                       w.tpart, tsl, r > 0 ? b : nullptr, (int)r, y);
  return hipGetLastError();
}

}  // namespace fp4rl
