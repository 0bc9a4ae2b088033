// Backward of the W4A16 linear with LoRA (gfx950).
//
// QeRL keeps the NVFP4 base frozen and trains only the low-rank adapters
// (QeRL explainer, "NVFP4 quantization and LoRA"), so for
// y = x deq(Wq)^T + s (x A^T) B^T the backward needs
//   dX = dY deq(Wq) + s (dY B) A,   dA = s (dY B)^T x,   dB = s dY^T (x A^T).
//
// Every product runs on one bf16 MFMA GEMM kernel whose operands are both
// contiguous along the contraction (nt_gemm_kernel), so the other operands
// are first laid out that way:
//   1. dequant_t_kernel: the tiled NVFP4 weight (codes contiguous along k)
//      -> Wt = g S_b as bf16 [K][N], exact (every g S_b has at most 6
//      significant bits).
//   2. transposes: B -> Bt [r][N]; A -> At2 [K][2 rp] = (A^T | A^T); dY and x
//      -> dYt [N][mp], Xt [K][mp], so that tokens become a contraction.
//   3. t = s x A^T and h = s dY B (contraction split over workgroups, fp32
//      partials), each summed and split into bf16 hi + lo (v = hi + lo to
//      ~2^-17 relative): tst, hst [2 rp][mp] and hs [M][2 rp].
//   4. dX = s_t dY Wt^T + (hi | lo of h) At2^T, one launch with two
//      contraction segments, rounded once to bf16.
//   5. dB = dYt (tst)^T and dA = hst Xt^T (token contraction split over
//      workgroups); fold_kernel adds the slices and the hi and lo halves.
#include <algorithm>

#include "backward.hpp"
#include "device.hpp"
#include "gemm_nt.hpp"

namespace fp4rl {
namespace {


// ---------------------------------------------------------------------------
// 1. Transposed dequantisation. A workgroup takes 4 row tiles (64 features)
// of one 128-k chunk: each wave dequantises one 1 KB tile (a lane holds row
// i, k = 32 j + 8 g .. + 7 of word j) into an LDS image [k][n], then the
// workgroup writes 128 rows of 64 features (128 B each) of Wt.
// ---------------------------------------------------------------------------
constexpr int kDtPitch = 72;  // bf16 per LDS row: 64 + 8

__global__ __launch_bounds__(256) void dequant_t_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, int N, int K,
                                                        uint16_t* __restrict__ wt) {
  __shared__ __align__(16) uint16_t tr[128 * kDtPitch];
  const int RT = (N + 15) >> 4, KC = (K + 127) >> 7;
  const int c = blockIdx.x, rg = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int rt = 4 * rg + w;
  if (rt < RT) {
    const int64_t tile = (int64_t)rt * KC + c;
    const uint4 v = *reinterpret_cast<const uint4*>(codes + tile * 1024 + 16 * lane);
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(scales + tile * 128 + 4 * (16 * (lg >> 1) + li));
    const uint32_t cw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 d = __builtin_bit_cast(uint4, dequant8(cw[j], e4m3_to_f32((sw >> (8 * j)) & 0xFFu)));
      const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
      uint16_t* col = tr + (32 * j + 8 * lg) * kDtPitch + 16 * w + li;
#pragma unroll
      for (int e = 0; e < 8; ++e) col[e * kDtPitch] = (uint16_t)(dw[e >> 1] >> (16 * (e & 1)));
    }
  }
  __syncthreads();
  const int row = threadIdx.x >> 1, h = threadIdx.x & 1;
  const int k = 128 * c + row;
  if (k >= K) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = 64 * rg + 32 * h + 8 * q;  // N % 8 == 0: a piece is all in or all out
    if (n < N)
      *reinterpret_cast<uint4*>(wt + (int64_t)k * N + n) =
          *reinterpret_cast<const uint4*>(tr + row * kDtPitch + 32 * h + 8 * q);
  }
}

// ---------------------------------------------------------------------------
// 2. out[c][col0 + i] = in[i][c] for i < rows, 0 for rows <= i < rows_pad;
// 64 x 64 tiles through LDS, both sides coalesced.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_u16_kernel(const uint16_t* __restrict__ in, int rows, int cols,
                                                            uint16_t* __restrict__ out, int ldo, int col0,
                                                            int rows_pad) {
  __shared__ uint16_t tl[64][65];
  const int c0 = 64 * blockIdx.x, r0 = 64 * blockIdx.y;
  for (int e = threadIdx.x; e < 4096; e += 256) {
    const int i = r0 + (e >> 6), cc = c0 + (e & 63);
    tl[e >> 6][e & 63] = (i < rows && cc < cols) ? in[(int64_t)i * cols + cc] : (uint16_t)0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 4096; e += 256) {
    const int i = r0 + (e & 63), cc = c0 + (e >> 6);
    if (cc < cols && i < rows_pad) out[(int64_t)cc * ldo + col0 + i] = tl[e & 63][e >> 6];
  }
}


// out[c][i] = in[i][c] with 16-byte accesses on both sides (cols, ldo and
// rows_pad multiples of 8); rows rows..rows_pad of out are zero.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ in, int rows, int cols,
                                                          uint16_t* __restrict__ out, int ldo, int rows_pad) {
  __shared__ __align__(16) uint16_t tl[64][66];
  const int c0 = 64 * blockIdx.x, r0 = 64 * blockIdx.y;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int e = threadIdx.x + 256 * p, i = e >> 3, cp = 8 * (e & 7);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + i < rows && c0 + cp < cols) v = *reinterpret_cast<const uint4*>(in + (int64_t)(r0 + i) * cols + c0 + cp);
    uint32_t* d = reinterpret_cast<uint32_t*>(&tl[i][cp]);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int e = threadIdx.x + 256 * p, cc = e >> 3, ip = 8 * (e & 7);
    if (c0 + cc < cols && r0 + ip < rows_pad) {
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = (uint32_t)tl[ip + 2 * t][cc] | ((uint32_t)tl[ip + 2 * t + 1][cc] << 16);
      *reinterpret_cast<uint4*>(out + (int64_t)(c0 + cc) * ldo + r0 + ip) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// 4. Finishing kernels (slices summed in order).
// rank_split_kernel: v = sum_s part[s][m][j] (m < M, j < r) split into bf16
//   hi + lo; written as sp [M][2 rp] (hi | lo) and/or spt [2 rp][mp]
//   (transposed, for contractions over tokens). Ranks r..rp and tokens
//   M..mp are zero.
// fold_kernel: out[a][b] = sum_s (part[s][a lda + b] + part[s][a lda + b + off]),
//   the hi and lo halves of a contraction against a split operand.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rank_split_kernel(const float* __restrict__ part, int slices, int M, int r,
                                                         int rp, int mp, uint16_t* __restrict__ sp,
                                                         uint16_t* __restrict__ spt) {
  const int64_t count = (int64_t)rp * mp;
  const int64_t sstride = (int64_t)M * r;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256) {
    const int j = (int)(e / mp), m = (int)(e - (int64_t)j * mp);  // tokens fastest: spt rows are contiguous
    float v = 0.0f;
    if (m < M && j < r)
      for (int s = 0; s < slices; ++s) v += part[s * sstride + (int64_t)m * r + j];
    const uint32_t hb = f32_to_bf16(v);
    const uint16_t hi = (uint16_t)hb, lo = (uint16_t)f32_to_bf16(v - __uint_as_float(hb << 16));
    if (spt) {
      spt[(int64_t)j * mp + m] = hi;
      spt[(int64_t)(rp + j) * mp + m] = lo;
    }
    if (sp && m < M) {
      sp[(int64_t)m * 2 * rp + j] = hi;
      sp[(int64_t)m * 2 * rp + rp + j] = lo;
    }
  }
}

__global__ __launch_bounds__(256) void fold_kernel(const float* __restrict__ part, int slices, int64_t sstride, int A,
                                                   int B, int lda, int64_t off, float* __restrict__ out) {
  const int64_t count = (int64_t)A * B;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (int64_t)gridDim.x * 256) {
    const int a = (int)(e / B), b = (int)(e - (int64_t)a * B);
    const int64_t i = (int64_t)a * lda + b;
    float v = 0.0f;
    for (int s = 0; s < slices; ++s) v += part[s * sstride + i] + part[s * sstride + i + off];
    out[e] = v;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

hipError_t launch_nt_bf16(Seg s1, Seg s2, int64_t m, int64_t q, const float* alpha_dev, uint16_t* y, hipStream_t st) {
  s1.slice = s1.c;
  // a 256 x 128 tile (WM = 2: 128 x 64 per wave, one workgroup per CU) measured slower than 128 x 128
  hipLaunchKernelGGL((nt_gemm_kernel<true, 1>), dim3((unsigned)nt_tiles(m, q)), dim3(256), 0, st, s1, s2, (int)m,
                     (int)q, alpha_dev, 0.0f, nullptr, y, nullptr);
  return hipGetLastError();
}

// fp32 partial products part[slice][m][q]; returns the number of slices
int launch_nt_part(Seg s1, int64_t m, int64_t q, float alpha, float* part, hipStream_t st) {
  const int64_t tiles = nt_tiles(m, q);
  s1.slice = nt_slice_len(tiles, s1.c);
  const int slices = nt_slices(tiles, s1.c);
  hipLaunchKernelGGL((nt_gemm_kernel<false, 1>), dim3((unsigned)tiles, (unsigned)slices), dim3(256), 0, st, s1, Seg{},
                     (int)m, (int)q, nullptr, alpha, nullptr, nullptr, part);
  return slices;
}

unsigned flat_grid(int64_t count) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((count + 255) / 256, 8192)); }

}  // namespace

// Workspace regions, in order, each 256-byte aligned (rp = r rounded up to 8,
// mp = m rounded up to 8):
//   Wt [k][n] bf16 (dX only); with adapters: Bt [r][n], At2 [k][2 rp] (dX
//   only), dYt [n][mp], Xt [k][mp], hs [m][2 rp] (dX only), hst and tst
//   [2 rp][mp] (bf16), and the fp32 slice partials of every split product.
size_t backward_workspace(int64_t m, int64_t n, int64_t k, int64_t r, bool want_dx, BackwardWs* w, void* base) {
  const int64_t rp = (r + 7) / 8 * 8, mp = (m + 7) / 8 * 8;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al256(bytes);
    return base ? static_cast<uint8_t*>(base) + o : nullptr;
  };
  BackwardWs v{};
  if (want_dx) v.wt = reinterpret_cast<uint16_t*>(take((size_t)k * n * 2));
  if (r > 0) {
    v.bt = reinterpret_cast<uint16_t*>(take((size_t)r * n * 2));
    if (want_dx) v.at2 = reinterpret_cast<uint16_t*>(take((size_t)k * 2 * rp * 2));
    v.dyt = reinterpret_cast<uint16_t*>(take((size_t)n * mp * 2));
    v.xt = reinterpret_cast<uint16_t*>(take((size_t)k * mp * 2));
    if (want_dx) v.hs = reinterpret_cast<uint16_t*>(take((size_t)m * 2 * rp * 2));
    v.hst = reinterpret_cast<uint16_t*>(take((size_t)2 * rp * mp * 2));
    v.tst = reinterpret_cast<uint16_t*>(take((size_t)2 * rp * mp * 2));
    // partials: t (x A^T), h (dY Bt^T), dB (dYt tst^T), dA (hst Xt^T)
    const size_t pt = (size_t)nt_slices(nt_tiles(m, r), k) * m * r;
    const size_t ph = (size_t)nt_slices(nt_tiles(m, r), n) * m * r;
    const size_t pb = (size_t)nt_slices(nt_tiles(n, 2 * rp), mp) * n * 2 * rp;
    const size_t pa = (size_t)nt_slices(nt_tiles(2 * rp, k), mp) * 2 * rp * k;
    v.part = reinterpret_cast<float*>(take(4 * std::max(std::max(pt, ph), std::max(pb, pa))));
  }
  if (w) *w = v;
  return off;
}

hipError_t launch_lora_backward(const uint16_t* dy, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                const uint16_t* a, const uint16_t* b, int64_t r, float s, uint16_t* dx, float* da,
                                float* db, const BackwardWs& w, hipStream_t st) {
  const int64_t rp = (r + 7) / 8 * 8, mp = (m + 7) / 8 * 8;
  hipError_t e = hipSuccess;
  if (dx) {
    const int64_t kc = (k + 127) / 128, rg = ((n + 15) / 16 + 3) / 4;
    hipLaunchKernelGGL(dequant_t_kernel, dim3((unsigned)kc, (unsigned)rg), dim3(256), 0, st, codes, scales, (int)n,
                       (int)k, w.wt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (r > 0) {
    hipLaunchKernelGGL(transpose_u16_kernel, dim3((unsigned)((r + 63) / 64), (unsigned)((n + 63) / 64)), dim3(256), 0,
                       st, b, (int)n, (int)r, w.bt, (int)n, 0, (int)n);
    if (dx)
      for (int half = 0; half < 2; ++half)
        hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)((k + 63) / 64), (unsigned)((rp + 63) / 64)), dim3(256),
                           0, st, a, (int)r, (int)k, w.at2 + half * rp, (int)(2 * rp), (int)rp);
    // tokens become the contraction of dA and dB: dY and x transposed, zero-padded to mp tokens
    hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)((n + 63) / 64), (unsigned)((mp + 63) / 64)), dim3(256), 0,
                       st, dy, (int)m, (int)n, w.dyt, (int)mp, (int)mp);
    hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)((k + 63) / 64), (unsigned)((mp + 63) / 64)), dim3(256), 0,
                       st, x, (int)m, (int)k, w.xt, (int)mp, (int)mp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // t = s x A^T -> tst (hi | lo, transposed)
    int sl = launch_nt_part(Seg{x, a, (int)k, (int)k}, m, r, s, w.part, st);
    hipLaunchKernelGGL(rank_split_kernel, dim3(flat_grid(rp * mp)), dim3(256), 0, st, w.part, sl, (int)m, (int)r,
                       (int)rp, (int)mp, nullptr, w.tst);
    // h = s dY B -> hst (transposed) and hs (for the LoRA segment of dX)
    sl = launch_nt_part(Seg{dy, w.bt, (int)n, (int)n}, m, r, s, w.part, st);
    hipLaunchKernelGGL(rank_split_kernel, dim3(flat_grid(rp * mp)), dim3(256), 0, st, w.part, sl, (int)m, (int)r,
                       (int)rp, (int)mp, dx ? w.hs : nullptr, w.hst);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (dx) {
    const Seg lora = r > 0 ? Seg{w.hs, w.at2, (int)(2 * rp), (int)(2 * rp)} : Seg{};
    if ((e = launch_nt_bf16(Seg{dy, w.wt, (int)n, (int)n}, lora, m, k, tensor_scale, dx, st)) != hipSuccess) return e;
  }
  if (r > 0) {
    // dB[n][j] = sum_m dY[m][n] t[m][j]: rows n of dYt against the 2 rp rows of tst, halves folded
    int sl = launch_nt_part(Seg{w.dyt, w.tst, (int)mp, (int)mp}, n, 2 * rp, 1.0f, w.part, st);
    hipLaunchKernelGGL(fold_kernel, dim3(flat_grid(n * r)), dim3(256), 0, st, w.part, sl, (int64_t)n * 2 * rp, (int)n,
                       (int)r, (int)(2 * rp), (int64_t)rp, db);
    // dA[j][k] = sum_m h[m][j] x[m][k]: the 2 rp rows of hst against rows k of Xt
    sl = launch_nt_part(Seg{w.hst, w.xt, (int)mp, (int)mp}, 2 * rp, k, 1.0f, w.part, st);
    hipLaunchKernelGGL(fold_kernel, dim3(flat_grid(r * k)), dim3(256), 0, st, w.part, sl, (int64_t)2 * rp * k, (int)r,
                       (int)k, (int)k, (int64_t)rp * k, da);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_zero_words(void* p, int64_t words, hipStream_t st) {
  if (words <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(flat_grid(words)), dim3(256), 0, st, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace fp4rl
