// Adaptive Quantization Noise RMSNorm for gfx950.
//
// QeRL explainer page, "Adaptive Quantization Noise (AQN)": the noise vector
// is folded into the RMSNorm scale, W_noise = Z_noise + w (the equation in
// "Zero overhead: integration into layer normalisation"), so channel-wise
// additive weight noise becomes row-wise multiplicative noise on the input
// of the next linear, and costs no extra parameters. The norm is read as the
// root-MEAN-square (the printed equation omits the 1/d).
//
// One launch per call. Each workgroup first regenerates the whole noise
// vector into LDS from a counter-based generator — Philox4x32-10 (Salmon,
// Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11)
// keyed by (seed, step, norm_id), then Box-Muller on 24-bit uniforms — so no
// RNG state and no workspace exist and every workgroup agrees bit for bit on
// the integers. Then one wave per row: 16-byte bf16 loads kept in registers,
// fp32 sum of squares, a DPP/shuffle wave reduction, one IEEE sqrt and
// division, and 16-byte bf16 stores. HBM traffic is 4 bytes per element.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace fp4rl {
namespace {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;
constexpr int kThreads = 256;
constexpr int kRowsPerWg = kThreads / kWave;
constexpr int kRegChunks = 16;  // 16-byte chunks per lane held in registers: d <= 8192

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t lo0 = kPhiloxM0 * c.x, hi0 = __umulhi(kPhiloxM0, c.x);
    const uint32_t lo1 = kPhiloxM1 * c.z, hi1 = __umulhi(kPhiloxM1, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return c;
}

// Two standard normals from two 32-bit words: u1 in (0,1], u2 in [0,1).
__device__ __forceinline__ void box_muller(uint32_t a, uint32_t b, float& zc, float& zs) {
  const float u1 = (float)((a >> 8) + 1u) * 0x1p-24f;
  const float u2 = (float)(b >> 8) * 0x1p-24f;
  const float rho = sqrtf(-2.0f * logf(u1));
  float s, c;
  sincospif(2.0f * u2, &s, &c);
  zc = rho * c;
  zs = rho * s;
}

__device__ __forceinline__ float sumsq8(uint4 v) {
  float a = bf16_lo(v.x), b = bf16_hi(v.x), c = bf16_lo(v.y), d = bf16_hi(v.y);
  float e = bf16_lo(v.z), f = bf16_hi(v.z), g = bf16_lo(v.w), h = bf16_hi(v.w);
  return ((a * a + b * b) + (c * c + d * d)) + ((e * e + f * f) + (g * g + h * h));
}

// (outputs rounded to bf16 by the hardware RNE convert, two per instruction)
__device__ __forceinline__ uint4 norm8(uint4 v, const float* wn, float inv) {
  const float4 w0 = *reinterpret_cast<const float4*>(wn);
  const float4 w1 = *reinterpret_cast<const float4*>(wn + 4);
  uint4 o;
  o.x = pack_bf16x2(bf16_lo(v.x) * inv * w0.x, bf16_hi(v.x) * inv * w0.y);
  o.y = pack_bf16x2(bf16_lo(v.y) * inv * w0.z, bf16_hi(v.y) * inv * w0.w);
  o.z = pack_bf16x2(bf16_lo(v.z) * inv * w1.x, bf16_hi(v.z) * inv * w1.y);
  o.w = pack_bf16x2(bf16_lo(v.w) * inv * w1.z, bf16_hi(v.w) * inv * w1.w);
  return o;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void aqn_rmsnorm_kernel(
    const uint16_t* __restrict__ x, int64_t m, int d, const float* __restrict__ w, float sigma,
    uint32_t seed_lo, uint32_t seed_hi, uint32_t step_lo, uint32_t step_hi, uint32_t norm_id,
    float eps, uint16_t* __restrict__ y, float* __restrict__ w_noise_out) {
  extern __shared__ float wn[];  // noisy weight, d floats (padded to a multiple of 8)

  const int nblocks = (d + 3) >> 2;
  for (int q = threadIdx.x; q < nblocks; q += kThreads) {
    const uint4 o = philox4x32_10(make_uint4((uint32_t)q, norm_id, step_lo, step_hi), seed_lo, seed_hi);
    float z[4];
    box_muller(o.x, o.y, z[0], z[1]);
    box_muller(o.z, o.w, z[2], z[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * q + j;
      if (i < d) {
        const float v = fmaf(sigma, z[j], w[i]);
        wn[i] = v;
        if (blockIdx.x == 0 && w_noise_out != nullptr) w_noise_out[i] = v;
      }
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const float inv_d = 1.0f / (float)d;
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerWg + wv; row < m; row += (int64_t)gridDim.x * kRowsPerWg) {
    const uint16_t* xr = x + row * d;
    uint16_t* yr = y + row * d;
    if constexpr (VEC) {
      const int nv = d >> 3;  // 16-byte chunks of 8 bf16
      const uint4* xv = reinterpret_cast<const uint4*>(xr);
      uint4* yv = reinterpret_cast<uint4*>(yr);
      uint4 reg[kRegChunks];
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < kRegChunks; ++c) {
        const int vi = lane + kWave * c;
        if (vi < nv) {
          reg[c] = ld_nt16(xv + vi);
          ss += sumsq8(reg[c]);
        }
      }
      for (int vi = lane + kWave * kRegChunks; vi < nv; vi += kWave) ss += sumsq8(xv[vi]);
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss * inv_d + eps);
#pragma unroll
      for (int c = 0; c < kRegChunks; ++c) {
        const int vi = lane + kWave * c;
        if (vi < nv) st_nt16(yv + vi, norm8(reg[c], wn + 8 * vi, inv));
      }
      for (int vi = lane + kWave * kRegChunks; vi < nv; vi += kWave) yv[vi] = norm8(xv[vi], wn + 8 * vi, inv);
    } else {
      float ss = 0.0f;
      for (int i = lane; i < d; i += kWave) {
        const float v = bf16_lo(xr[i]);
        ss += v * v;
      }
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss * inv_d + eps);
      for (int i = lane; i < d; i += kWave) yr[i] = (uint16_t)f32_to_bf16(bf16_lo(xr[i]) * inv * wn[i]);
    }
  }
}

// Few rows (decode batches): the noise of d columns would cost each
// workgroup far more than its rows, so workgroups split the columns instead.
// Workgroup (slice, group) makes the noise of its kColSlice columns only
// (wave 0), while each of its waves loads one full row into registers — the
// same row is loaded by every slice, mostly from L2 — sums its squares in the
// same lane order and wave reduction as the row kernel above (so both give
// the same result), and writes its slice of the row from those registers.
constexpr int kColSlice = 256;  // columns per workgroup (64 Philox blocks)

__global__ __launch_bounds__(kThreads) void aqn_rmsnorm_cols_kernel(
    const uint16_t* __restrict__ x, int m, int d, const float* __restrict__ w, float sigma, uint32_t seed_lo,
    uint32_t seed_hi, uint32_t step_lo, uint32_t step_hi, uint32_t norm_id, float eps, uint16_t* __restrict__ y,
    float* __restrict__ w_noise_out) {
  __shared__ __align__(16) float wn[kColSlice];
  const int col0 = blockIdx.x * kColSlice;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int row = blockIdx.y * kRowsPerWg + wv;
  const int nv = d >> 3;  // 16-byte chunks of 8 bf16 per row
  // this wave's row, first kRegChunks chunks per lane in registers
  uint4 reg[kRegChunks];
  float ss = 0.0f;
  const uint4* xv = reinterpret_cast<const uint4*>(x + (int64_t)min(row, max(m - 1, 0)) * d);
  if (row < m) {
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
      const int vi = lane + kWave * c;
      if (vi < nv) reg[c] = xv[vi];
    }
  }
  if (threadIdx.x < kColSlice / 4) {
    const int q = col0 / 4 + threadIdx.x;  // Philox block of columns 4 q .. 4 q + 3
    const uint4 o = philox4x32_10(make_uint4((uint32_t)q, norm_id, step_lo, step_hi), seed_lo, seed_hi);
    float z[4];
    box_muller(o.x, o.y, z[0], z[1]);
    box_muller(o.z, o.w, z[2], z[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * q + j;
      const float v = i < d ? fmaf(sigma, z[j], w[i]) : 0.0f;
      wn[4 * threadIdx.x + j] = v;
      if (i < d && blockIdx.y == 0 && w_noise_out != nullptr) w_noise_out[i] = v;
    }
  }
  __syncthreads();
  if (row >= m) return;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c)
    if (lane + kWave * c < nv) ss += sumsq8(reg[c]);
  for (int vi = lane + kWave * kRegChunks; vi < nv; vi += kWave) ss += sumsq8(xv[vi]);
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / (float)d) + eps);
  uint4* yv = reinterpret_cast<uint4*>(y + (int64_t)row * d);
  const int v0 = col0 / 8, v1 = min(nv, v0 + kColSlice / 8);  // this slice's chunks
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int vi = lane + kWave * c;
    if (vi >= v0 && vi < v1) yv[vi] = norm8(reg[c], wn + 8 * (vi - v0), inv);
  }
  for (int vi = lane + kWave * kRegChunks; vi < v1; vi += kWave)  // rows wider than the registers hold
    if (vi >= v0) yv[vi] = norm8(xv[vi], wn + 8 * (vi - v0), inv);
}

__global__ void philox_words_kernel(uint32_t seed_lo, uint32_t seed_hi, uint32_t step_lo,
                                    uint32_t step_hi, uint32_t norm_id, int64_t n_blocks,
                                    uint4* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q < n_blocks) out[q] = philox4x32_10(make_uint4((uint32_t)q, norm_id, step_lo, step_hi), seed_lo, seed_hi);
}

}  // namespace

hipError_t launch_aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, const float* w, float sigma,
                              uint64_t seed, uint64_t step, uint32_t norm_id, float eps,
                              uint16_t* y, float* w_noise_out, hipStream_t stream) {
  const bool vec = (d % 8) == 0;
  const uint32_t sl0 = (uint32_t)seed, sh0 = (uint32_t)(seed >> 32);
  const uint32_t tl0 = (uint32_t)step, th0 = (uint32_t)(step >> 32);
  if (vec && m <= 256) {  // few rows: split the columns (and the noise) over workgroups
    // m == 0 still runs one row group: the noisy weight is written even without rows
    const dim3 grid((unsigned)((d + kColSlice - 1) / kColSlice),
                    (unsigned)std::max<int64_t>(1, (m + kRowsPerWg - 1) / kRowsPerWg));
    hipLaunchKernelGGL(aqn_rmsnorm_cols_kernel, grid, dim3(kThreads), 0, stream, x, (int)m, (int)d, w, sigma, sl0,
                       sh0, tl0, th0, norm_id, eps, y, w_noise_out);
    return hipGetLastError();
  }
  const int64_t rows_wg = (m + kRowsPerWg - 1) / kRowsPerWg;
  // Enough workgroups to fill 256 CUs several times over (eight per CU) while
  // the per-workgroup noise prologue (d/4 Philox blocks) stays small next to
  // the rows: 65536 x 5120 takes 286 us with 2048 workgroups, 327 with 1024
  // and 316 with 4096.
  int64_t grid = std::max<int64_t>(1, std::min<int64_t>(rows_wg, 2048));
  const size_t lds = (size_t)((d + 7) / 8) * 8 * sizeof(float);
  const uint32_t sl = (uint32_t)seed, sh = (uint32_t)(seed >> 32);
  const uint32_t tl = (uint32_t)step, th = (uint32_t)(step >> 32);
  if (vec)
    hipLaunchKernelGGL(aqn_rmsnorm_kernel<true>, dim3((unsigned)grid), dim3(kThreads), lds, stream, x, m,
                       (int)d, w, sigma, sl, sh, tl, th, norm_id, eps, y, w_noise_out);
  else
    hipLaunchKernelGGL(aqn_rmsnorm_kernel<false>, dim3((unsigned)grid), dim3(kThreads), lds, stream, x, m,
                       (int)d, w, sigma, sl, sh, tl, th, norm_id, eps, y, w_noise_out);
  return hipGetLastError();
}

hipError_t launch_philox_words(uint64_t seed, uint64_t step, uint32_t norm_id, int64_t n_blocks,
                               uint32_t* out, hipStream_t stream) {
  const int64_t grid = (n_blocks + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(philox_words_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, (uint32_t)seed,
                     (uint32_t)(seed >> 32), (uint32_t)step, (uint32_t)(step >> 32), norm_id, n_blocks,
                     reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace fp4rl
