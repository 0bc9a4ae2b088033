// Backward of the W4A16 linear with LoRA (gfx950).
//
// QeRL keeps the NVFP4 base frozen and trains only the low-rank adapters
// (QeRL explainer, "NVFP4 quantization and LoRA"), so for
// y = x deq(Wq)^T + s (x A^T) B^T the backward needs
//   dX = dY deq(Wq) + s (dY B) A,   dA = s (dY B)^T x,   dB = s dY^T (x A^T).
//
// The contraction of dX runs over the output features n, across the rows of
// the tiled weight, whose codes are contiguous along k. Work is split as:
//   1. dequant_t_kernel: the tiled NVFP4 weight -> Wt = g S_b as bf16 [K][N]
//      (exact: every g S_b has at most 6 significant bits), one pass.
//   2. transpose_u16_kernel: B -> Bt [r][N]; A -> At2 [K][2 rp] = (A^T | A^T),
//      rank columns r..rp zero.
//   3. nt_gemm_kernel (bf16 MFMA 16x16x32, fp32 accumulate): with both
//      operands contiguous along the contraction,
//        t = s x A^T     [M][r] fp32,
//        h = s dY Bt^T   [M][r] fp32, also split into bf16 hi | lo [M][2 rp],
//        dX = s_t dY Wt^T + (hi | lo) At2^T, rounded once to bf16.
//      The LoRA term of dX is a second contraction segment of the same
//      kernel; the hi + lo split keeps h to ~2^-17 relative.
//   4. tn_grad_kernel (fp32 VALU, M split over workgroups, slices summed in
//      order by reduce_kernel): dA = h^T x, dB = dY^T t.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace fp4rl {
namespace {

constexpr int kRsrcWord3 = 0x00020000;

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

// ---------------------------------------------------------------------------
// 3. C[m][q] = alpha sum_c L1[m][c] R1[q][c] (+ sum_c L2[m][c] R2[q][c]), bf16
// operands with rows contiguous along c (c % 8 == 0), fp32 accumulation.
// A workgroup computes a 128 (m) x 128 (q) tile with 4 waves of 64 x 64
// (4 x 4 MFMA tiles each). Contraction chunks of 64 are loaded to registers
// one chunk ahead and written to one of two LDS slabs per operand (rows
// padded to 144 B: conflict-free 16-byte fragment reads); one barrier per
// chunk. Rows past M or Q are clamped (loaded, never stored); pieces past c
// read as zero through the buffer descriptor's range.
// A lane's result holds q = 4 g + v of MFMA column li = m, so stores are
// 4 consecutive outputs of one row.
// ---------------------------------------------------------------------------
constexpr int kGT = 128, kGC = 64, kGPitch = kGC + 8;

struct Seg {
  const uint16_t* l = nullptr;  // [M][c]
  const uint16_t* r = nullptr;  // [Q][c]
  int c = 0;                    // contraction length (0: no segment)
};

template <bool BF16OUT>
__global__ __launch_bounds__(256) void nt_gemm_kernel(Seg s1, Seg s2, int M, int Q, const float* __restrict__ alpha_dev,
                                                      float alpha, uint16_t* __restrict__ ybf, float* __restrict__ yf,
                                                      uint16_t* __restrict__ ysplit, int rp) {
  __shared__ __align__(16) uint16_t ls[2][kGT * kGPitch];
  __shared__ __align__(16) uint16_t rs[2][kGT * kGPitch];
  const int MT = (M + kGT - 1) / kGT;
  const int mt = blockIdx.x % MT, qt = blockIdx.x / MT;
  const int m0 = kGT * mt, q0 = kGT * qt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave & 1, wq = wave >> 1;
  const int prow = threadIdx.x >> 3, pcol = threadIdx.x & 7;  // piece: rows prow + 32 i, bf16 8 pcol .. + 7

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto run = [&](const Seg& S) {
    const int C = S.c, NC = (C + kGC - 1) / kGC;
    const int lrows = min(kGT, M - m0), rrows = min(kGT, Q - q0);
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(S.l + (int64_t)m0 * C), 0, 2 * lrows * C, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(S.r + (int64_t)q0 * C), 0, 2 * rrows * C, kRsrcWord3);
    uint32_t loff[4], roff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      loff[i] = 2u * ((uint32_t)min(prow + 32 * i, lrows - 1) * (uint32_t)C + 8 * pcol);
      roff[i] = 2u * ((uint32_t)min(prow + 32 * i, rrows - 1) * (uint32_t)C + 8 * pcol);
    }
    uint4 lv[4], rv[4];
    auto load = [&](int ch) {
      ch = min(ch, NC - 1);
      const uint32_t out = kGC * ch + 8 * pcol < C ? 0u : 0x80000000u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lrs, (int)((loff[i] + 2u * kGC * ch) | out), 0, 0));
        rv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rrs, (int)((roff[i] + 2u * kGC * ch) | out), 0, 0));
      }
    };
    auto store = [&](int slab) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&ls[slab][(prow + 32 * i) * kGPitch + 8 * pcol]) = lv[i];
        *reinterpret_cast<uint4*>(&rs[slab][(prow + 32 * i) * kGPitch + 8 * pcol]) = rv[i];
      }
    };
    __syncthreads();  // the slabs of a previous segment are no longer read
    load(0);
    store(0);
    load(1);
    for (int ch = 0; ch < NC; ++ch) {
      __syncthreads();  // slab ch % 2 is complete; the other is no longer read
      if (ch + 1 < NC) {
        store((ch + 1) & 1);
        load(ch + 2);
      }
      const uint16_t* lsl = ls[ch & 1];
      const uint16_t* rsl = rs[ch & 1];
#pragma unroll
      for (int st = 0; st < kGC / 32; ++st) {
        bf16x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = as_bf16x8(*reinterpret_cast<const uint4*>(rsl + (64 * wq + 16 * i + li) * kGPitch + 32 * st + 8 * lg));
          b[i] = as_bf16x8(*reinterpret_cast<const uint4*>(lsl + (64 * wm + 16 * i + li) * kGPitch + 32 * st + 8 * lg));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
      }
    }
  };

  run(s1);
  const float al = alpha_dev ? *alpha_dev : alpha;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] *= al;
  if (s2.c > 0) run(s2);

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + 64 * wm + 16 * j + li, q = q0 + 64 * wq + 16 * i + 4 * lg;
      if (m >= M) continue;
      const f32x4 v = acc[i][j];
      if constexpr (BF16OUT) {
        uint16_t* yp = ybf + (int64_t)m * Q + q;
        if (q + 3 < Q) {  // Q % 4 == 0 here (Q = K, a multiple of 16)
          *reinterpret_cast<uint2*>(yp) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (q + e < Q) yp[e] = (uint16_t)f32_to_bf16(v[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (q + e < Q) yf[(int64_t)m * Q + q + e] = v[e];
          if (ysplit && q + e < rp) {
            const float f = q + e < Q ? v[e] : 0.0f;
            const uint32_t hb = f32_to_bf16(f);
            ysplit[(int64_t)m * 2 * rp + q + e] = (uint16_t)hb;
            ysplit[(int64_t)m * 2 * rp + rp + q + e] = (uint16_t)f32_to_bf16(f - __uint_as_float(hb << 16));
          }
        }
      }
    }
}

// ---------------------------------------------------------------------------
// 4. part[slice][p][q] = sum over the slice's rows m of L[m][p] R[m][q]
// (fp32 FMA, rows in order). 64 x 64 output tiles, 16 rows of each operand
// per step staged in LDS as fp32; a thread owns 4 x 4 outputs.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float ld_f32(const T* p, int64_t i) {
  if constexpr (sizeof(T) == 2) return __uint_as_float((uint32_t)p[i] << 16);  // bf16
  else return p[i];
}

template <typename TL, typename TR>
__global__ __launch_bounds__(256) void tn_grad_kernel(const TL* __restrict__ L, int P, const TR* __restrict__ R, int Q,
                                                      int M, int mslice, float* __restrict__ part) {
  __shared__ __align__(16) float lsh[16][64];
  __shared__ __align__(16) float rsh[16][64];
  const int PT = (P + 63) / 64;
  const int pt = blockIdx.x % PT, qt = blockIdx.x / PT;
  const int p0 = 64 * pt, q0 = 64 * qt;
  const int mb = blockIdx.y * mslice, me = min(M, mb + mslice);
  const int tp = threadIdx.x >> 4, tq = threadIdx.x & 15;
  const int er = threadIdx.x >> 4, ec = 4 * (threadIdx.x & 15);
  float acc[4][4] = {};
  for (int m0 = mb; m0 < me; m0 += 16) {
    const int m = m0 + er;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = p0 + ec + j, q = q0 + ec + j;
      lsh[er][ec + j] = (m < me && p < P) ? ld_f32(L, (int64_t)m * P + p) : 0.0f;
      rsh[er][ec + j] = (m < me && q < Q) ? ld_f32(R, (int64_t)m * Q + q) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) {
      const float4 lv = *reinterpret_cast<const float4*>(&lsh[mm][4 * tp]);
      const float4 rv = *reinterpret_cast<const float4*>(&rsh[mm][4 * tq]);
      const float l4[4] = {lv.x, lv.y, lv.z, lv.w}, r4[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(l4[a], r4[b], acc[a][b]);
    }
    __syncthreads();
  }
  float* out = part + (int64_t)blockIdx.y * P * Q;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int p = p0 + 4 * tp + a;
    if (p >= P) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int q = q0 + 4 * tq + b;
      if (q < Q) out[(int64_t)p * Q + q] = acc[a][b];
    }
  }
}

// out[i] = sum_s part[s][i], slices in order
__global__ __launch_bounds__(256) void slice_sum_kernel(const float* __restrict__ part, int slices, int64_t count,
                                                        float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    float v = 0.0f;
    for (int s = 0; s < slices; ++s) v += part[(int64_t)s * count + i];
    out[i] = v;
  }
}

int grad_slices(int64_t m, int64_t p, int64_t q) {
  const int64_t tiles = ((p + 63) / 64) * ((q + 63) / 64);
  int64_t s = (1024 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, m / 256));
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, 32));
}

int grad_mslice(int64_t m, int slices) { return (int)(((m + slices - 1) / slices + 15) / 16 * 16); }

size_t al256(size_t v) { return (v + 255) / 256 * 256; }

template <typename TL, typename TR>
hipError_t launch_tn(const TL* L, int64_t p, const TR* R, int64_t q, int64_t m, float* part, float* out,
                     hipStream_t st) {
  const int slices0 = grad_slices(m, p, q);
  const int mslice = grad_mslice(m, slices0);
  const int slices = (int)((m + mslice - 1) / mslice);
  const unsigned tiles = (unsigned)(((p + 63) / 64) * ((q + 63) / 64));
  float* dst = slices > 1 ? part : out;
  hipLaunchKernelGGL((tn_grad_kernel<TL, TR>), dim3(tiles, (unsigned)slices), dim3(256), 0, st, L, (int)p, R, (int)q,
                     (int)m, mslice, dst);
  if (slices > 1) {
    const int64_t count = p * q;
    const unsigned grid = (unsigned)std::min<int64_t>((count + 255) / 256, 4096);
    hipLaunchKernelGGL(slice_sum_kernel, dim3(grid), dim3(256), 0, st, part, slices, count, out);
  }
  return hipGetLastError();
}

hipError_t launch_nt(bool bf16out, Seg s1, Seg s2, int64_t m, int64_t q, const float* alpha_dev, float alpha,
                     uint16_t* ybf, float* yf, uint16_t* ysplit, int64_t rp, hipStream_t st) {
  const unsigned grid = (unsigned)(((m + kGT - 1) / kGT) * ((q + kGT - 1) / kGT));
  if (bf16out)
    hipLaunchKernelGGL(nt_gemm_kernel<true>, dim3(grid), dim3(256), 0, st, s1, s2, (int)m, (int)q, alpha_dev, alpha,
                       ybf, yf, ysplit, (int)rp);
  else
    hipLaunchKernelGGL(nt_gemm_kernel<false>, dim3(grid), dim3(256), 0, st, s1, s2, (int)m, (int)q, alpha_dev, alpha,
                       ybf, yf, ysplit, (int)rp);
  return hipGetLastError();
}

}  // namespace

// Workspace regions, in order, each 256-byte aligned:
//   Wt [k][n] bf16 (only with dX), Bt [r][n] bf16, At2 [k][2 rp] bf16,
//   t [m][r] fp32, h [m][r] fp32, hs [m][2 rp] bf16, slice partials fp32.
size_t backward_workspace(int64_t m, int64_t n, int64_t k, int64_t r, bool want_dx, BackwardWs* w, void* base) {
  const int64_t rp = (r + 7) / 8 * 8;
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
    v.t = reinterpret_cast<float*>(take((size_t)m * r * 4));
    v.h = reinterpret_cast<float*>(take((size_t)m * r * 4));
    if (want_dx) v.hs = reinterpret_cast<uint16_t*>(take((size_t)m * 2 * rp * 2));
    const int sa = grad_slices(m, r, k), sb = grad_slices(m, n, r);
    const size_t pa = sa > 1 ? (size_t)sa * r * k * 4 : 0, pb = sb > 1 ? (size_t)sb * n * r * 4 : 0;
    if (pa || pb) v.part = reinterpret_cast<float*>(take(std::max(pa, pb)));
  }
  if (w) *w = v;
  return off;
}

hipError_t launch_lora_backward(const uint16_t* dy, const uint16_t* x, int64_t m, int64_t n, int64_t k,
                                const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                const uint16_t* a, const uint16_t* b, int64_t r, float s, uint16_t* dx, float* da,
                                float* db, const BackwardWs& w, hipStream_t st) {
  const int64_t rp = (r + 7) / 8 * 8;
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
        hipLaunchKernelGGL(transpose_u16_kernel, dim3((unsigned)((k + 63) / 64), (unsigned)((rp + 63) / 64)),
                           dim3(256), 0, st, a, (int)r, (int)k, w.at2, (int)(2 * rp), (int)(half * rp), (int)rp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // t = s x A^T, h = s dY B (and its bf16 hi | lo split for the dX segment)
    if ((e = launch_nt(false, Seg{x, a, (int)k}, Seg{}, m, r, nullptr, s, nullptr, w.t, nullptr, 0, st)) != hipSuccess)
      return e;
    if ((e = launch_nt(false, Seg{dy, w.bt, (int)n}, Seg{}, m, r, nullptr, s, nullptr, w.h, dx ? w.hs : nullptr, rp,
                       st)) != hipSuccess)
      return e;
  }
  if (dx) {
    const Seg lora = r > 0 ? Seg{w.hs, w.at2, (int)(2 * rp)} : Seg{};
    if ((e = launch_nt(true, Seg{dy, w.wt, (int)n}, lora, m, k, tensor_scale, 0.0f, dx, nullptr, nullptr, 0, st)) !=
        hipSuccess)
      return e;
  }
  if (r > 0) {
    if ((e = launch_tn<float, uint16_t>(w.h, r, x, k, m, w.part, da, st)) != hipSuccess) return e;  // dA = h^T x
    if ((e = launch_tn<uint16_t, float>(dy, n, w.t, r, m, w.part, db, st)) != hipSuccess) return e;  // dB = dY^T t
  }
  return hipSuccess;
}

hipError_t launch_zero_words(void* p, int64_t words, hipStream_t st) {
  if (words <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((words + 255) / 256, 4096);
  hipLaunchKernelGGL(slice_sum_kernel, dim3(grid), dim3(256), 0, st, nullptr, 0, words, static_cast<float*>(p));
  return hipGetLastError();
}

}  // namespace fp4rl
