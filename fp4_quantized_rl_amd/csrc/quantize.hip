// NVFP4 block quantiser for gfx950.
//
// Follows the QeRL explainer page ("NVFP4 quantization and LoRA": frozen
// weights held in 4-bit NVFP4) and the TRACE article ("Engineering view of
// the mechanism": a small group of values shares one scale and each value
// rounds up or down to a neighbouring grid point). Format: 16-element blocks
// along K, one OCP E4M3 scale byte per block, one fp32 tensor scale, E2M1
// codes packed two per byte (even element in the low nibble).
//
// Two HBM-bound passes, because the global amax is a true dependency of
// every block scale:
//   1. amax_kernel: grid-stride |w| max as uint32 bit patterns (exact and
//      order-free for non-negative floats); one partial per workgroup.
//   2. encode_kernel (row-major output) / encode_tiled_kernel (tiled
//      output): every workgroup reduces the partials to amax itself (no
//      atomics, no memset, no third launch), then each quad of lanes owns
//      one 16-element block: 16-byte loads, quad max by two xor shuffles,
//      E4M3 byte, and 16 exact nearest-even E2M1 codes. The tiled variant
//      assembles whole tiles in LDS and writes them with 16-byte stores.
// Exactness: every comparison of |x| with a grid midpoint m*D is the sign of
// fmaf(m, D, -|x|); the exact difference is 0 or at least 2^-149 in
// magnitude once D >= 2^-100 (blocks with smaller D are rescaled by 2^64,
// exactly), so the fused result has the exact sign.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace fp4rl {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ uint32_t absbits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// |.| maximum of one 16-byte vector, as fp32 bit patterns.
template <bool BF16>
__device__ __forceinline__ uint32_t vec_absmax(uint4 v) {
  if constexpr (BF16) {
    uint32_t m = max(max((v.x << 16) & 0x7FFF0000u, v.x & 0x7FFF0000u),
                     max((v.y << 16) & 0x7FFF0000u, v.y & 0x7FFF0000u));
    return max(m, max(max((v.z << 16) & 0x7FFF0000u, v.z & 0x7FFF0000u),
                      max((v.w << 16) & 0x7FFF0000u, v.w & 0x7FFF0000u)));
  } else {
    return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint4* __restrict__ w, int64_t nvec,
                                                         uint32_t* __restrict__ partial) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t mx = 0;
  for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = w[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mx = max(mx, vec_absmax<BF16>(v[u]));
  }
  for (; i < nvec; i += stride) mx = max(mx, vec_absmax<BF16>(w[i]));
  mx = wave_max_u32(mx);
  __shared__ uint32_t red[kThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
#pragma unroll
    for (int j = 1; j < kThreads / kWave; ++j) m = max(m, red[j]);
    partial[blockIdx.x] = m;
  }
}

// Nearest E4M3 byte to r >= 0, ties to even, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float r) {
  if (!(r < 448.0f)) return 0x7Eu;
  if (r < 0x1p-6f) return (uint32_t)__builtin_rintf(r * 512.0f);  // subnormal grid m*2^-9; 8 -> 0x08
  uint32_t b = __float_as_uint(r);
  b += 0x7FFFFu + ((b >> 20) & 1u);  // round the 23-bit mantissa to 3 bits, half to even
  return min((b >> 20) - (120u << 3), 0x7Eu);
}

// E2M1 code of x for block step D (Ds = D or D*2^64, xs = 1 or 2^64).
// E2M1 code of x for block scale D (Ds = D, or D * 2^64 with xs = 2^64 for
// tiny D). The magnitude index k is the number of grid midpoints m_i * D
// (m = 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) that |x| passes, where a tie goes
// to the even index: |x| must exceed the midpoints below an odd index
// (0.25, 1.25, 2.5, 5) and reach those below an even one (0.75, 1.75, 3.5).
// The passes are monotone in |x|, so k is found by binary search: three
// exact sign tests instead of seven.
__device__ __forceinline__ uint32_t e2m1_encode(float x, bool dzero, float Ds, float xs) {
#pragma clang fp contract(off)
  const float ax = fabsf(x) * xs;
  const bool t4 = fmaf(1.75f, Ds, -ax) <= 0.0f;  // k >= 4
  const bool t2 = fmaf(t4 ? 3.5f : 0.75f, Ds, -ax) <= 0.0f;  // k >= 4 t4 + 2
  const float mlo = t4 ? (t2 ? 5.0f : 2.5f) : (t2 ? 1.25f : 0.25f);
  const bool t1 = fmaf(mlo, Ds, -ax) < 0.0f;  // k odd
  uint32_t k = 4u * (uint32_t)t4 + 2u * (uint32_t)t2 + (uint32_t)t1;
  k = dzero ? 0u : k;
  return k | ((__float_as_uint(x) >> 28) & 8u);
}

// Rounding record (TRACE article, "Engineering view of the mechanism": each
// value is rounded up or down to a neighbouring grid point, and the rollout
// side records that choice): 1 when the chosen grid point g_k * D exceeds |x|
// (the magnitude was rounded up), by the same exact sign test as the
// midpoints; 0 when rounded down or hit exactly, and for D == 0.
__device__ __forceinline__ uint32_t e2m1_rounded_up(uint32_t code, float x, bool dzero, float Ds, float xs) {
#pragma clang fp contract(off)
  const uint32_t k = code & 7u;
  const float g = k < 4u ? 0.5f * (float)k : (k == 7u ? 6.0f : (float)(k - 2u));
  return (!dzero && fmaf(g, Ds, -(fabsf(x) * xs)) > 0.0f) ? 1u : 0u;
}

template <bool BF16>
__device__ __forceinline__ void load_quarter(const void* w, int64_t idx, float v[4]) {
  if constexpr (BF16) {
    const uint2 r = ld_nt8(reinterpret_cast<const uint2*>(w) + idx);
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x); v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
  } else {
    const uint4 r = ld_nt16(reinterpret_cast<const uint4*>(w) + idx);
    v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y); v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
  }
}

// Destination of block b's two code bytes of quarter q and of its scale byte.
// Row-major: codes [n][k/2], scales [n][k/16]. Tiled: 16-row x 128-k tiles
// (1 KB of codes + 128 B of scales each, tile (rt, c) at rt*kc + c). Inside a
// tile, lane l = 16 g + i of a wave finds its 16 code bytes at 16 l, word j of
// them holding row i, k = 128 c + 32 j + 8 g .. + 7; the scale word 16 p + i
// holds in byte j the scale of block 8 c + 2 j + p. So a block kb (8 per
// chunk) lands in word j = kb/2 of lane groups g = 2 (kb & 1) and g + 1, and
// its quarter q (4 elements) in group g + q/2, byte 2 (q & 1) of the word.
template <bool BF16, bool REC>
__global__ __launch_bounds__(kThreads) void encode_kernel(const void* __restrict__ w, int64_t nblk,
                                                           const uint32_t* __restrict__ partial,
                                                           int npartial, uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           float* __restrict__ tensor_scale,
                                                           uint8_t* __restrict__ record) {
#pragma clang fp contract(off)
  __shared__ uint32_t red[kThreads / kWave];
  uint32_t mx = 0;
  for (int i = threadIdx.x; i < npartial; i += kThreads) mx = max(mx, partial[i]);
  mx = wave_max_u32(mx);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int j = 1; j < kThreads / kWave; ++j) mx = max(mx, red[j]);
  const float st = __uint_as_float(mx) / 2688.0f;  // IEEE division
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = st;
  const float six_st = 6.0f * st;

  const int q = threadIdx.x & 3;  // quarter of the block this lane holds
  const int64_t nquads = (int64_t)gridDim.x * (kThreads / 4);
  for (int64_t b0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / 4; b0 < nblk; b0 += kUnroll * nquads) {
    float v[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t b = b0 + u * nquads;
      if (b < nblk) load_quarter<BF16>(w, 4 * b + q, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t b = b0 + u * nquads;
      if (b >= nblk) break;  // uniform across the quad
      uint32_t ab = max(max(absbits(v[u][0]), absbits(v[u][1])), max(absbits(v[u][2]), absbits(v[u][3])));
      ab = max(ab, (uint32_t)__shfl_xor((int)ab, 1, kWave));
      ab = max(ab, (uint32_t)__shfl_xor((int)ab, 2, kWave));
      const float a_b = __uint_as_float(ab);
      const uint32_t byte = (st != 0.0f && a_b != 0.0f) ? e4m3_encode(a_b / six_st) : 0u;
      const float D = e4m3_to_f32(byte) * st;
      const bool tiny = D < 0x1p-100f;
      const float Ds = tiny ? D * 0x1p64f : D;
      const float xs = tiny ? 0x1p64f : 1.0f;
      const bool dz = D == 0.0f;
      const uint32_t c = e2m1_encode(v[u][0], dz, Ds, xs) | (e2m1_encode(v[u][1], dz, Ds, xs) << 4) |
                         (e2m1_encode(v[u][2], dz, Ds, xs) << 8) | (e2m1_encode(v[u][3], dz, Ds, xs) << 12);
      // row-major: the block's 8 code bytes, then its scale byte
      *reinterpret_cast<uint16_t*>(codes + 8 * b + 2 * q) = (uint16_t)c;
      if (q == 0) scales[b] = (uint8_t)byte;
      if constexpr (REC) {  // this quarter's 4 bits; the even lane of a pair stores the byte
        uint32_t nib = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) nib |= e2m1_rounded_up(c >> (4 * e), v[u][e], dz, Ds, xs) << e;
        const uint32_t other = (uint32_t)__shfl_xor((int)nib, 1, kWave);
        if ((q & 1) == 0) record[2 * b + (q >> 1)] = (uint8_t)(nib | (other << 4));
      }
    }
  }
}

// Tiled output: one workgroup encodes a region of 16 rows (one row tile) x
// kRegionChunks 128-wide K chunks, i.e. whole tiles, into an LDS image of
// those tiles, then writes them with 16-byte stores: each tile's 1 KB of
// codes and 128 B of scales are contiguous, and consecutive chunks of a row
// tile are consecutive tiles, so the region is one contiguous run. (Writing
// each lane's share straight to the tiled layout touched eight 64-byte
// lines per store instruction and cost 18% of the encode pass.)
// Two lanes share a block, eight elements each: the block max takes one xor
// shuffle, the E4M3 byte is computed once per eight elements, and the eight
// codes are one 4-byte word of the tile (word j of lane slot (g, i)). Pair
// (row i, r) takes blocks r, r + 8, r + 16, r + 24 of the region's row i; a
// wave's load instruction covers 4 rows x 128 contiguous elements.
// Elements past N or K (padding) encode as zero codes with a zero scale
// byte, so the tiled buffers need no separate fill.
constexpr int kRegionChunks = 4;
constexpr int kRegionBlocks = 8 * kRegionChunks;  // per row
constexpr int kBlocksPerPair = kRegionBlocks / 8;

template <bool BF16>
__device__ __forceinline__ void load_half(const void* w, int64_t elem, float v[8]) {
  if constexpr (BF16) {
    const uint4 r = ld_nt16(reinterpret_cast<const uint16_t*>(w) + elem);
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x); v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
    v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z); v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
  } else {
    const float* p = reinterpret_cast<const float*>(w) + elem;
    const uint4 a = ld_nt16(p), b = ld_nt16(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

template <bool BF16, bool REC>
__global__ __launch_bounds__(kThreads) void encode_tiled_kernel(const void* __restrict__ w, int n, int k,
                                                                 const uint32_t* __restrict__ partial, int npartial,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales,
                                                                 float* __restrict__ tensor_scale,
                                                                 uint8_t* __restrict__ record) {
#pragma clang fp contract(off)
  __shared__ uint32_t red[kThreads / kWave];
  __shared__ __align__(16) uint8_t img[kRegionChunks * (1024 + 128)];  // codes of the region's tiles, then scales
  uint32_t mx = 0;
  for (int i = threadIdx.x; i < npartial; i += kThreads) mx = max(mx, partial[i]);
  mx = wave_max_u32(mx);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int j = 1; j < kThreads / kWave; ++j) mx = max(mx, red[j]);
  const float st = __uint_as_float(mx) / 2688.0f;  // IEEE division
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = st;
  const float six_st = 6.0f * st;

  const int h = threadIdx.x & 1, pd = threadIdx.x >> 1;  // half of the block, pair
  const int i = pd >> 3, r = pd & 7;                     // row within the tile, pair within the row
  const int kc = (k + 127) >> 7, kblocks = k >> 4;
  const int ngroups = (kc + kRegionChunks - 1) / kRegionChunks;
  const int64_t regions = (int64_t)((n + 15) >> 4) * ngroups;
  for (int64_t reg = blockIdx.x; reg < regions; reg += gridDim.x) {
    const int rt = (int)(reg / ngroups), cg = (int)(reg - (int64_t)rt * ngroups);
    const int row = 16 * rt + i, kb0 = kRegionBlocks * cg;
    float v[kBlocksPerPair][8];
#pragma unroll
    for (int u = 0; u < kBlocksPerPair; ++u) {
      const int kb = kb0 + r + 8 * u;
      if (row < n && kb < kblocks) {
        load_half<BF16>(w, (int64_t)row * k + 16 * kb + 8 * h, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kBlocksPerPair; ++u) {
      uint32_t ab = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) ab = max(ab, absbits(v[u][e]));
      ab = max(ab, (uint32_t)__shfl_xor((int)ab, 1, kWave));
      const float a_b = __uint_as_float(ab);
      const uint32_t byte = (st != 0.0f && a_b != 0.0f) ? e4m3_encode(a_b / six_st) : 0u;
      const float D = e4m3_to_f32(byte) * st;
      const bool tiny = D < 0x1p-100f;
      const float Ds = tiny ? D * 0x1p64f : D;
      const float xs = tiny ? 0x1p64f : 1.0f;
      const bool dz = D == 0.0f;
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) c |= e2m1_encode(v[u][e], dz, Ds, xs) << (4 * e);
      // tiled position of this half block (block kb of row i: tile kb / 8, kq = kb % 8)
      const int kbl = r + 8 * u, t = kbl >> 3, kq = kbl & 7, p = kq & 1, j = kq >> 1;
      const int g = 2 * p + h;
      *reinterpret_cast<uint32_t*>(img + 1024 * t + 16 * (16 * g + i) + 4 * j) = c;
      if (h == 0) img[kRegionChunks * 1024 + 128 * t + 4 * (16 * p + i) + j] = (uint8_t)byte;
      if constexpr (REC) {  // row-major record: this half block is byte 2 kb + h of the row
        const int kb = kb0 + kbl;
        if (row < n && kb < kblocks) {
          uint32_t bits = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) bits |= e2m1_rounded_up(c >> (4 * e), v[u][e], dz, Ds, xs) << e;
          record[(int64_t)row * (k >> 3) + 2 * kb + h] = (uint8_t)bits;
        }
      }
    }
    __syncthreads();
    const int tiles = min(kRegionChunks, kc - kRegionChunks * cg);  // tiles of this region inside the matrix
    const int64_t tile0 = (int64_t)rt * kc + kRegionChunks * cg;
    if ((int)threadIdx.x < 64 * tiles)
      *reinterpret_cast<uint4*>(codes + tile0 * 1024 + 16 * threadIdx.x) =
          *reinterpret_cast<const uint4*>(img + 16 * threadIdx.x);
    if ((int)threadIdx.x < 32 * tiles)
      *reinterpret_cast<uint32_t*>(scales + tile0 * 128 + 4 * threadIdx.x) =
          *reinterpret_cast<const uint32_t*>(img + kRegionChunks * 1024 + 4 * threadIdx.x);
    __syncthreads();  // the image is rewritten by the next region
  }
}

__global__ void write_zero_scale(float* tensor_scale) { *tensor_scale = 0.0f; }

// Zero fill (the padding of tiled buffers); a kernel rather than a memset so
// that captured graphs hold only kernel nodes.
__global__ void to_tiled_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int N, int K,
                                int kc, int64_t pieces, uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= pieces) return;
  const int lane = (int)(p & 63), g = lane >> 4, i = lane & 15;
  const int64_t tile = p >> 6;
  const int rt = (int)(tile / kc), c = (int)(tile - (int64_t)rt * kc);
  const int n = 16 * rt + i;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  uint32_t sv = 0;
  if (n < N) {
    const uint8_t* cr = codes + (int64_t)n * (K / 2);
    const uint8_t* sr = scales + (int64_t)n * (K / 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k0 = 128 * c + 32 * j + 8 * g;  // 8 codes = 4 bytes, 4-byte aligned (K % 16 == 0)
      if (k0 < K) w[j] = *reinterpret_cast<const uint32_t*>(cr + k0 / 2);
      if (g < 2) {
        const int kb = 8 * c + 2 * j + g;  // scale word p = g
        if (16 * kb < K) sv |= (uint32_t)sr[kb] << (8 * j);
      }
    }
  }
  *reinterpret_cast<uint4*>(codes_t + tile * 1024 + 16 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
  if (g < 2) *reinterpret_cast<uint32_t*>(scales_t + tile * 128 + 4 * (16 * g + i)) = sv;
}

}  // namespace

size_t quantize_workspace_bytes() { return kAmaxPartials * sizeof(uint32_t); }

int64_t nvfp4_codes_bytes(int64_t n, int64_t k, bool tiled) {
  return tiled ? ((n + 15) / 16) * ((k + 127) / 128) * 1024 : n * k / 2;
}

int64_t nvfp4_scales_bytes(int64_t n, int64_t k, bool tiled) {
  return tiled ? ((n + 15) / 16) * ((k + 127) / 128) * 128 : n * k / 16;
}

hipError_t launch_quantize(const void* w, bool w_bf16, int64_t n, int64_t k, bool tiled, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, uint8_t* record, uint32_t* partial,
                           hipStream_t stream) {
  const int64_t elems = n * k;
  if (elems == 0) {
    hipLaunchKernelGGL(write_zero_scale, dim3(1), dim3(1), 0, stream, tensor_scale);
    return hipGetLastError();
  }
  const int64_t nvec = elems / (w_bf16 ? 8 : 4);  // k % 16 == 0, so vectors never straddle
  const int64_t g1 = std::min<int64_t>(kAmaxPartials, std::max<int64_t>(1, (nvec + kThreads * kUnroll - 1) / (kThreads * kUnroll)));
  if (w_bf16)
    hipLaunchKernelGGL(amax_kernel<true>, dim3((unsigned)g1), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(w), nvec, partial);
  else
    hipLaunchKernelGGL(amax_kernel<false>, dim3((unsigned)g1), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(w), nvec, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nblk = elems / 16;
  const int64_t per_wg = (kThreads / 4) * kUnroll;
  const dim3 grid((unsigned)std::min<int64_t>(8192, (nblk + per_wg - 1) / per_wg));
  if (tiled) {  // whole tiles per workgroup (padding written as zero)
    const int64_t regions = ((n + 15) / 16) * ((k / 128 + (k % 128 != 0) + kRegionChunks - 1) / kRegionChunks);
    const dim3 tgrid((unsigned)std::min<int64_t>(8192, regions));
#define FP4RL_TILED(B_, R_)                                                                                  \
  hipLaunchKernelGGL((encode_tiled_kernel<B_, R_>), tgrid, dim3(kThreads), 0, stream, w, (int)n, (int)k, partial, \
                     (int)g1, codes, scales, tensor_scale, record)
    if (w_bf16) {
      if (record) FP4RL_TILED(true, true); else FP4RL_TILED(true, false);
    } else {
      if (record) FP4RL_TILED(false, true); else FP4RL_TILED(false, false);
    }
#undef FP4RL_TILED
    return hipGetLastError();
  }
#define FP4RL_ROWS(B_, R_)                                                                                    \
  hipLaunchKernelGGL((encode_kernel<B_, R_>), grid, dim3(kThreads), 0, stream, w, nblk, partial, (int)g1, codes, \
                     scales, tensor_scale, record)
  if (w_bf16) {
    if (record) FP4RL_ROWS(true, true); else FP4RL_ROWS(true, false);
  } else {
    if (record) FP4RL_ROWS(false, true); else FP4RL_ROWS(false, false);
  }
#undef FP4RL_ROWS
  return hipGetLastError();
}

hipError_t launch_to_tiled(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, uint8_t* codes_t,
                           uint8_t* scales_t, hipStream_t stream) {
  const int64_t kc = (k + 127) / 128;
  const int64_t pieces = ((n + 15) / 16) * kc * 64;
  hipLaunchKernelGGL(to_tiled_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, codes, scales,
                     (int)n, (int)k, (int)kc, pieces, codes_t, scales_t);
  return hipGetLastError();
}

}  // namespace fp4rl
