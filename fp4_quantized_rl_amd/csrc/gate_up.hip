// Gate and up projections of one input in one launch, with the SiLU-gated
// product as epilogue (gfx950), for decode batches (M <= 128).
//
// The Qwen2.5 models that QeRL trains (QeRL explainer, experiments) gate
// their MLP: h = SiLU(gate) * up, where gate and up are two linears of the
// same input. Here both are NVFP4 + LoRA linears (own weights, tensor scale
// and adapters), and
//   h = bf16(SiLU(g) * u),  g = s_tg acc_g + tg . Bg[n],  u = s_tu acc_u + tu . Bu[n],
// with g and u kept in fp32 (one rounding, of h), SiLU(v) = v / (1 + e^-v).
//
// gate_up_kernel<T, RT>: one workgroup per RT 16-row weight tiles of BOTH
// matrices (the same output features n); its four waves take the 128-k
// chunks in turn. Per chunk a lane loads 16 code bytes and 4 scale bytes of each tile
// (word j of the tiled layout: row i, k = 32 j + 8 g .. + 7) and, for each of
// the T token tiles, its 16-byte token fragments (token i, the same k), and
// issues 4 x T MFMAs per matrix. Each wave scales its sums by the tensor
// scales; waves 0 and 1 add the gate's and the up's LoRA terms by MFMA (t in
// bf16 hi + lo against the B rows); the four waves' sums are added in wave
// order through LDS, and every thread takes outputs in turn for the gated
// product.
// t_g = s x Ag^T and t_u = s x Au^T come from the linear's LoRA
// down-projection kernel.
#include <algorithm>

#include "device.hpp"
#include "gate_up.hpp"
#include "lora_mfma.hpp"
#include "launch.hpp"

namespace fp4rl {
namespace {

// the four OCP E4M3 bytes of w as fp32 (exact)
__device__ __forceinline__ void e4m3_scales(uint32_t w, float (&sc)[4]) {
  sc[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
  sc[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  sc[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
  sc[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}

// One 8-value token fragment of x, optionally normalised on the way in:
// bf16((x r_m) w_k), the AQN RMSNorm's rounding and order of operations
// (r_m = 1 / sqrt(mean x^2 + eps), w = w + sigma z the noisy weight).
template <bool NORM>
__device__ __forceinline__ uint4 token_fragment(const uint16_t* p, float rinv, const float* wn) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  if constexpr (!NORM) {
    return v;
  } else {
    const float4 w0 = *reinterpret_cast<const float4*>(wn), w1 = *reinterpret_cast<const float4*>(wn + 4);
    return make_uint4(pack_bf16x2(bf16_lo(v.x) * rinv * w0.x, bf16_hi(v.x) * rinv * w0.y),
                      pack_bf16x2(bf16_lo(v.y) * rinv * w0.z, bf16_hi(v.y) * rinv * w0.w),
                      pack_bf16x2(bf16_lo(v.z) * rinv * w1.x, bf16_hi(v.z) * rinv * w1.y),
                      pack_bf16x2(bf16_lo(v.w) * rinv * w1.z, bf16_hi(v.w) * rinv * w1.w));
  }
}

// PAIR = false: one projection only (the gate's arguments), h = bf16(g).
template <int T, int RT, bool NORM = false, bool PAIR = true>
__global__ __launch_bounds__(256) void gate_up_kernel(const uint16_t* __restrict__ x, int M, int N, int K,
                                                      const uint8_t* __restrict__ cg, const uint8_t* __restrict__ sg,
                                                      const float* __restrict__ stg, const uint8_t* __restrict__ cu,
                                                      const uint8_t* __restrict__ su, const float* __restrict__ stu,
                                                      const float* __restrict__ tg, const float* __restrict__ tu,
                                                      int tsl, const uint16_t* __restrict__ bg,
                                                      const uint16_t* __restrict__ bu, int r,
                                                      uint16_t* __restrict__ h, const float* __restrict__ wn,
                                                      const float* __restrict__ rinv) {
  constexpr int P = PAIR ? 2 : 1;  // projections
  __shared__ f32x4 red[4][P * RT * T][64];
  extern __shared__ float wns[];  // NORM: the noisy norm weight, K floats (dynamic LDS)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (NORM) {
    for (int i = 4 * threadIdx.x; i < K; i += 1024)  // K % 16 == 0
      *reinterpret_cast<float4*>(wns + i) = *reinterpret_cast<const float4*>(wn + i);
    __syncthreads();
  }
  const int li = lane & 15, lg = lane >> 4;
  const int KC = (K + 127) >> 7, NT = (N + 15) >> 4;
  const uint8_t *gcode[RT], *ucode[RT], *gsc[RT], *usc[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {  // row tiles past the matrix are clamped (never stored)
    const int64_t tile0 = (int64_t)min(RT * (int)blockIdx.x + i, NT - 1) * KC;
    gcode[i] = cg + tile0 * 1024 + 16 * lane;
    gsc[i] = sg + tile0 * 128 + 4 * (16 * (lg >> 1) + li);
    ucode[i] = PAIR ? cu + tile0 * 1024 + 16 * lane : nullptr;
    usc[i] = PAIR ? su + tile0 * 128 + 4 * (16 * (lg >> 1) + li) : nullptr;
  }
  const uint16_t* xrow[T];  // tokens past M are clamped (their columns are never stored)
  float rv[T];
#pragma unroll
  for (int j = 0; j < T; ++j) {
    xrow[j] = x + (int64_t)min(16 * j + li, M - 1) * K + 8 * lg;
    rv[j] = NORM ? rinv[min(16 * j + li, M - 1)] : 1.0f;
  }
  f32x4 ag[RT][T], au[RT][T];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < T; ++j) ag[i][j] = au[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = wave; c < KC; c += 4) {
    uint4 wg[RT], wu[RT] = {};
    uint32_t sgw[RT], suw[RT] = {};
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      wg[i] = ld_nt16(gcode[i] + (int64_t)c * 1024);
      sgw[i] = *reinterpret_cast<const uint32_t*>(gsc[i] + (int64_t)c * 128);
      if constexpr (PAIR) {
        wu[i] = ld_nt16(ucode[i] + (int64_t)c * 1024);
        suw[i] = *reinterpret_cast<const uint32_t*>(usc[i] + (int64_t)c * 128);
      }
    }
    uint4 xv[4][T];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int k = 128 * c + 32 * st + 8 * lg;  // K % 16 == 0: 8 values all in or all out
#pragma unroll
      for (int j = 0; j < T; ++j)
        xv[st][j] = k < K ? token_fragment<NORM>(xrow[j] + 128 * c + 32 * st, rv[j], wns + k) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const uint32_t cwg[4] = {wg[i].x, wg[i].y, wg[i].z, wg[i].w}, cwu[4] = {wu[i].x, wu[i].y, wu[i].z, wu[i].w};
      float scg[4], scu[4];
      e4m3_scales(sgw[i], scg);
      if constexpr (PAIR) e4m3_scales(suw[i], scu);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 a_g = dequant8(cwg[st], scg[st]);
#pragma unroll
        for (int j = 0; j < T; ++j) ag[i][j] = mfma16x16x32(a_g, as_bf16x8(xv[st][j]), ag[i][j]);
        if constexpr (PAIR) {
          const bf16x8 a_u = dequant8(cwu[st], scu[st]);
#pragma unroll
          for (int j = 0; j < T; ++j) au[i][j] = mfma16x16x32(a_u, as_bf16x8(xv[st][j]), au[i][j]);
        }
      }
    }
  }
  // each wave's partial sums times the tensor scales; the LoRA terms are
  // added by MFMA, the gate's by wave 0 and the up's by wave 1
  const float sgt = *stg, sut = PAIR ? *stu : 0.0f;
#pragma unroll
  for (int i = 0; i < RT; ++i) {
#pragma unroll
    for (int j = 0; j < T; ++j) {
      ag[i][j] *= sgt;
      au[i][j] *= sut;
    }
    if (r > 0 && wave == 0) lora_mfma<T>(ag[i], tg, tsl, bg, r, M, N, RT * (int)blockIdx.x + i, li, lg);
    if (PAIR && r > 0 && wave == 1) lora_mfma<T>(au[i], tu, tsl, bu, r, M, N, RT * (int)blockIdx.x + i, li, lg);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      red[wave][(P * i) * T + j][lane] = ag[i][j];
      if constexpr (PAIR) red[wave][(P * i + 1) * T + j][lane] = au[i][j];
    }
  }
  __syncthreads();
  // output e = (row tile i, token tl, feature row rl): the four waves' sums
  // in wave order, then the gated product
  for (int e = threadIdx.x; e < 256 * RT * T; e += 256) {
    const int i = e / (256 * T), el = e - i * 256 * T;
    const int tl = el >> 4, rl = el & 15;
    const int m = tl, n = 16 * (RT * (int)blockIdx.x + i) + rl;
    if (m >= M || n >= N) continue;
    const int j = tl >> 4, ln = 16 * (rl >> 2) + (tl & 15), v = rl & 3;
    const int sg_ = (P * i) * T + j;
    const float g = ((red[0][sg_][ln][v] + red[1][sg_][ln][v]) + red[2][sg_][ln][v]) + red[3][sg_][ln][v];
    if constexpr (PAIR) {
      const int su_ = (P * i + 1) * T + j;
      const float u = ((red[0][su_][ln][v] + red[1][su_][ln][v]) + red[2][su_][ln][v]) + red[3][su_][ln][v];
      h[(int64_t)m * N + n] = (uint16_t)f32_to_bf16(g / (1.0f + expf(-g)) * u);
    } else {
      h[(int64_t)m * N + n] = (uint16_t)f32_to_bf16(g);
    }
  }
}

// The AQN RMSNorm folded into the LoRA down-projections of gate and up (nad
// = 2) or of one projection (nad = 1): one workgroup per 16-token tile,
// 16-rank tile, adapter and K-slice (blockIdx.z = nad slice + adapter). Its waves first take 4 tokens each for their sum of
// squares (16-byte loads, all issued before the sums; r_m = 1 / sqrt(ss / K
// + eps), the norm's formula; the (., 0, 0) workgroup writes r_m for the
// projections), then take the slice's 32-k steps in turn, loading all their
// fragments before the MFMAs: A operand = adapter row li (k = 32 s + 8 g ..
// + 7), B operand = the normalised token fragment; the waves' sums are
// added in wave order into t's K-slice. With r == 0 only r_m is made.
// t = s xn A^T in K-slices; xn is never stored.
constexpr int kNormLoraSteps = 4;  // 32-k steps per wave and slice (at most)

__global__ __launch_bounds__(256) void norm_lora_down_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                             const float* __restrict__ wn, float eps,
                                                             const uint16_t* __restrict__ ag,
                                                             const uint16_t* __restrict__ au, int r, float s,
                                                             int kslice, float* __restrict__ rinv,
                                                             float* __restrict__ tg, float* __restrict__ tu,
                                                             int nad) {
  __shared__ float rs[16];
  __shared__ f32x4 red[3][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int m0 = 16 * blockIdx.x, j0 = 16 * blockIdx.y;
  const int adapter = nad == 2 ? (int)(blockIdx.z & 1) : 0, z = (int)blockIdx.z / nad;
  const int nv = K >> 3;  // 16-byte pieces per token row
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c = lane; c < nv; c += 64) {
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = *reinterpret_cast<const uint4*>(x + (int64_t)min(m0 + 4 * wave + q, M - 1) * K + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w4[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(w4[e]), hi = bf16_hi(w4[e]);
        ss[q] += lo * lo;
        ss[q] += hi * hi;
      }
    }
  }
  const float inv_k = 1.0f / (float)K;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float t = wave_sum(ss[q]);
    if (lane == 0) rs[4 * wave + q] = 1.0f / sqrtf(t * inv_k + eps);
  }
  __syncthreads();
  if (blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < 16 && m0 + (int)threadIdx.x < M)
    rinv[m0 + threadIdx.x] = rs[threadIdx.x];
  if (r == 0) return;
  const uint16_t* a = adapter == 0 ? ag : au;
  float* t = (adapter == 0 ? tg : tu) + (int64_t)z * M * r;
  const uint16_t* arow = a + (int64_t)min(j0 + li, r - 1) * K + 8 * lg;
  const uint16_t* xrow = x + (int64_t)min(m0 + li, M - 1) * K + 8 * lg;
  const float rm = rs[li];
  const int k0 = z * kslice, k1 = min(K, k0 + kslice);
  uint4 av[kNormLoraSteps], xv[kNormLoraSteps];
#pragma unroll
  for (int u = 0; u < kNormLoraSteps; ++u) {
    const int k = k0 + 32 * (wave + 4 * u) + 8 * lg;  // K % 16 == 0: 8 values all in or all out
    const bool in = k < k1;                            // lanes past the slice give zero operands
    av[u] = in ? *reinterpret_cast<const uint4*>(arow + k - 8 * lg) : make_uint4(0u, 0u, 0u, 0u);
    xv[u] = in ? token_fragment<true>(xrow + k - 8 * lg, rm, wn + k) : make_uint4(0u, 0u, 0u, 0u);
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kNormLoraSteps; ++u) acc = mfma16x16x32(as_bf16x8(av[u]), as_bf16x8(xv[u]), acc);
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
  acc = ((acc + red[0][lane]) + red[1][lane]) + red[2][lane];
  // lane holds ranks j0 + 4 g + v of token m0 + li
  const int m = m0 + li;
  if (m >= M) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int j = j0 + 4 * lg + v;
    if (j < r) t[(int64_t)m * r + j] = s * acc[v];
  }
}

// K-slices of the normalising LoRA down-projection: 4 waves x 4 steps of 32
int norm_lora_slices(int64_t k) { return (int)((k + 32 * 4 * kNormLoraSteps - 1) / (32 * 4 * kNormLoraSteps)); }

}  // namespace

int gate_up_token_tiles(int64_t m) { return m <= 16 ? 1 : m <= 32 ? 2 : m <= 64 ? 4 : 8; }

hipError_t launch_gate_up(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* cg, const uint8_t* sg,
                          const float* stg, const uint8_t* cu, const uint8_t* su, const float* stu,
                          const uint16_t* ag, const uint16_t* bg, const uint16_t* au, const uint16_t* bu, int64_t r,
                          float s, float* ws, uint16_t* h, hipStream_t st) {
  float *tg = nullptr, *tu = nullptr;
  int tsl = 0;
  if (r > 0) {  // t = s x A^T in K-slices
    const int splits = lora_splits(m, k, r);
    tsl = lora_slices(k, splits);
    const size_t part = ((size_t)tsl * m * r + 63) / 64 * 64;
    tg = ws;
    tu = ws + part;
    hipError_t e = launch_lora_down(x, m, k, ag, r, s, splits, tg, st);
    if (e == hipSuccess) e = launch_lora_down(x, m, k, au, r, s, splits, tu, st);
    if (e == hipSuccess && m > 16 && tsl > 1) {
      // more than one token tile: the slices are added once, in order, by a
      // reduction launch (up to 16 tokens the kernel adds them itself)
      float* sg_ = ws + 2 * part;
      float* su_ = sg_ + ((size_t)m * r + 63) / 64 * 64;
      e = launch_lora_reduce(tg, tsl, m * r, sg_, st);
      if (e == hipSuccess) e = launch_lora_reduce(tu, tsl, m * r, su_, st);
      tg = sg_;
      tu = su_;
      tsl = 1;
    }
    if (e != hipSuccess) return e;
  }
  const int T = gate_up_token_tiles(m);
  const int RT = T == 1 ? 1 : 2;  // row tiles per workgroup: two share each token fragment from 17 tokens on
  const dim3 grid((unsigned)(((n + 15) / 16 + RT - 1) / RT));
#define FP4RL_GATE_UP(TT, RR)                                                                                        \
  hipLaunchKernelGGL((gate_up_kernel<TT, RR>), grid, dim3(256), 0, st, x, (int)m, (int)n, (int)k, cg, sg, stg, cu, \
                     su, stu, tg, tu, tsl, bg, bu, (int)r, h, nullptr, nullptr)
  if (T == 1) FP4RL_GATE_UP(1, 1);
  else if (T == 2) FP4RL_GATE_UP(2, 2);
  else if (T == 4) FP4RL_GATE_UP(4, 2);
  else FP4RL_GATE_UP(8, 2);
#undef FP4RL_GATE_UP
  return hipGetLastError();
}

// h = bf16(SiLU(g) * u) from two bf16 linear outputs: the same fp32 formula
// as the fused epilogue; eight elements per thread and step (count % 8
// elements through the scalar tail)
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
                                                       int64_t count, uint16_t* __restrict__ h) {
  const int64_t n8 = count / 8, stride = (int64_t)gridDim.x * 256;
  auto f = [](float gv, float uv) { return gv / (1.0f + expf(-gv)) * uv; };
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    const uint4 gv = reinterpret_cast<const uint4*>(g)[i], uv = reinterpret_cast<const uint4*>(u)[i];
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = pack_bf16x2(f(bf16_lo(gw[j]), bf16_lo(uw[j])), f(bf16_hi(gw[j]), bf16_hi(uw[j])));
    reinterpret_cast<uint4*>(h)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  for (int64_t i = 8 * n8 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride)
    h[i] = (uint16_t)f32_to_bf16(f(bf16_lo(g[i]), bf16_lo(u[i])));
}

hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, int64_t count, uint16_t* h, hipStream_t st) {
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((count / 8 + 255) / 256, 2048));
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)blocks), dim3(256), 0, st, g, u, count, h);
  return hipGetLastError();
}

// [t_g K-slices][t_u K-slices] and, above 16 tokens with K split, [t_g][t_u] summed (fp32)
size_t gate_up_workspace(int64_t m, int64_t k, int64_t r) {
  if (r <= 0) return 0;
  const int tsl = lora_slices(k, lora_splits(m, k, r));
  const size_t part = ((size_t)tsl * m * r + 63) / 64 * 64, one = ((size_t)m * r + 63) / 64 * 64;
  return 4 * (2 * part + (m > 16 && tsl > 1 ? 2 * one : 0));
}

// [w_noise: k][r_m: m][t_g K-slices: S m r][t_u K-slices: S m r] (fp32, each 256-byte aligned)
size_t aqn_gate_up_workspace(int64_t m, int64_t k, int64_t r) {
  auto a = [](size_t v) { return (v * 4 + 255) / 256 * 256; };
  return a((size_t)k) + a((size_t)m) + 2 * a((size_t)norm_lora_slices(k) * m * r);
}

hipError_t launch_aqn_gate_up(const uint16_t* x, int64_t m, int64_t n, int64_t k, const float* norm_w, float sigma,
                              uint64_t seed, uint64_t step, uint32_t norm_id, float eps, const uint8_t* cg,
                              const uint8_t* sg, const float* stg, const uint8_t* cu, const uint8_t* su,
                              const float* stu, const uint16_t* ag, const uint16_t* bg, const uint16_t* au,
                              const uint16_t* bu, int64_t r, float s, void* ws, uint16_t* h, hipStream_t st) {
  auto a = [](size_t v) { return (v * 4 + 255) / 256 * 256; };
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* wn = reinterpret_cast<float*>(base);
  float* rinv = reinterpret_cast<float*>(base + a((size_t)k));
  const int S = norm_lora_slices(k);
  float* tg = reinterpret_cast<float*>(base + a((size_t)k) + a((size_t)m));
  float* tu = reinterpret_cast<float*>(base + a((size_t)k) + a((size_t)m) + a((size_t)S * m * r));
  // the noisy norm weight w + sigma z (no rows: the norm kernel's noise prologue alone)
  hipError_t e = launch_aqn_rmsnorm(nullptr, 0, k, norm_w, sigma, seed, step, norm_id, eps, nullptr, wn, st);
  if (e != hipSuccess) return e;
  const dim3 lgrid((unsigned)((m + 15) / 16), (unsigned)(r > 0 ? (r + 15) / 16 : 1), r > 0 ? 2u * S : 1u);
  hipLaunchKernelGGL(norm_lora_down_kernel, lgrid, dim3(256), 0, st, x, (int)m, (int)k, wn, eps, ag, au, (int)r, s,
                     32 * 4 * kNormLoraSteps, rinv, tg, tu, 2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int T = gate_up_token_tiles(m);
  // LDS: the waves' sums (8 KB per row tile and token tile) plus k floats of
  // the noisy weight (<= 64 KB): one row tile at 8 token tiles keeps it <= 128 KB
  const int RT = T == 1 || T == 8 ? 1 : 2;
  const dim3 grid((unsigned)(((n + 15) / 16 + RT - 1) / RT));
  const int tsl = r > 0 ? S : 0;
#define FP4RL_AQN_GATE_UP(TT, RR)                                                                                   \
  hipLaunchKernelGGL((gate_up_kernel<TT, RR, true>), grid, dim3(256), (size_t)k * 4, st, x, (int)m, (int)n, (int)k, cg, \
                     sg, stg, \
                     cu, su, stu, tg, tu, tsl, bg, bu, (int)r, h, wn, rinv)
  if (T == 1) FP4RL_AQN_GATE_UP(1, 1);
  else if (T == 2) FP4RL_AQN_GATE_UP(2, 2);
  else if (T == 4) FP4RL_AQN_GATE_UP(4, 2);
  else FP4RL_AQN_GATE_UP(8, 1);
#undef FP4RL_AQN_GATE_UP
  return hipGetLastError();
}

// [w_noise: k][r_m: m][t K-slices: S m r] (fp32, each 256-byte aligned)
size_t aqn_linear_workspace(int64_t m, int64_t k, int64_t r) {
  auto a = [](size_t v) { return (v * 4 + 255) / 256 * 256; };
  return a((size_t)k) + a((size_t)m) + a((size_t)norm_lora_slices(k) * m * r);
}

hipError_t launch_aqn_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const float* norm_w, float sigma,
                             uint64_t seed, uint64_t step, uint32_t norm_id, float eps, const uint8_t* codes,
                             const uint8_t* scales, const float* ts, const uint16_t* a, const uint16_t* b, int64_t r,
                             float s, void* ws, uint16_t* y, hipStream_t st) {
  auto al = [](size_t v) { return (v * 4 + 255) / 256 * 256; };
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* wn = reinterpret_cast<float*>(base);
  float* rinv = reinterpret_cast<float*>(base + al((size_t)k));
  float* t = reinterpret_cast<float*>(base + al((size_t)k) + al((size_t)m));
  const int S = norm_lora_slices(k);
  hipError_t e = launch_aqn_rmsnorm(nullptr, 0, k, norm_w, sigma, seed, step, norm_id, eps, nullptr, wn, st);
  if (e != hipSuccess) return e;
  const dim3 lgrid((unsigned)((m + 15) / 16), (unsigned)(r > 0 ? (r + 15) / 16 : 1), r > 0 ? (unsigned)S : 1u);
  hipLaunchKernelGGL(norm_lora_down_kernel, lgrid, dim3(256), 0, st, x, (int)m, (int)k, wn, eps, a, nullptr, (int)r, s,
                     32 * 4 * kNormLoraSteps, rinv, t, nullptr, 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int T = gate_up_token_tiles(m);
  // LDS: the waves' sums (4 KB per row tile and token tile) plus k floats of
  // the noisy weight (<= 64 KB)
  const int RT = T == 1 ? 1 : 2;
  const dim3 grid((unsigned)(((n + 15) / 16 + RT - 1) / RT));
  const int tsl = r > 0 ? S : 0;
#define FP4RL_AQN_LINEAR(TT, RR)                                                                                     \
  hipLaunchKernelGGL((gate_up_kernel<TT, RR, true, false>), grid, dim3(256), (size_t)k * 4, st, x, (int)m, (int)n,    \
                     (int)k, codes, scales, ts, nullptr, nullptr, nullptr, t, nullptr, tsl, b, nullptr, (int)r, y, wn, \
                     rinv)
  if (T == 1) FP4RL_AQN_LINEAR(1, 1);
  else if (T == 2) FP4RL_AQN_LINEAR(2, 2);
  else if (T == 4) FP4RL_AQN_LINEAR(4, 2);
  else FP4RL_AQN_LINEAR(8, 2);
#undef FP4RL_AQN_LINEAR
  return hipGetLastError();
}

}  // namespace fp4rl
