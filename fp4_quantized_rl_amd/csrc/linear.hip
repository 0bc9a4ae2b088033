// W4A16 NVFP4 linear with the fused LoRA update, for gfx950.
//
// QeRL explainer page, "NVFP4 quantization and LoRA" and "Experimental
// details": rollout runs the frozen NVFP4 base with 16-bit activations
// through a W4A16 kernel (Marlin on the pages' hardware), plus the trainable
// low-rank update. Computed here:
//
//   t = lora_scale * x A^T                       (lora_down_kernel, fp32)
//   y = bf16( s_t * sum_k x g(code) S_b  +  t B^T )   (skinny_kernel)
//
// Decode (small M) is bound by the weight stream: 0.5625 byte per weight
// (nibble + 1/16 scale byte). skinny_kernel streams codes with 16-byte loads
// (one lane = 32 consecutive k of one row = two blocks), dequantises in
// registers (hardware E2M1 convert at unit scale, times the E4M3 block
// scale: exact in bf16) and feeds v_mfma_f32_16x16x32_bf16 with the weights
// as the 16-row A operand and up to 8 tiles of 16 tokens as B operands. The
// K dimension is split across the waves of a workgroup and reduced through
// LDS (deterministic, no atomics); the LoRA up-projection runs in the
// epilogue as extra MFMA steps, with t split into bf16 hi + lo parts.
//
// Within one MFMA the order of the 32 k values is free as long as A and B
// use the same one, so a lane's 16-byte code load (k = 32g .. 32g+31 of a
// 128-wide chunk, g = lane/16) supplies its slot in four consecutive MFMAs.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace fp4rl {
namespace {

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// ---------------------------------------------------------------------------
// LoRA down-projection: t[m][j] = s * sum_k x[m][k] A[j][k].
// One workgroup per 16x16 tile of t; its waves split K and reduce in LDS.
// ---------------------------------------------------------------------------
template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void lora_down_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                   const uint16_t* __restrict__ a, int r, float s,
                                                                   float* __restrict__ t) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.x * 16, j0 = blockIdx.y * 16;
  const int m = m0 + li, j = j0 + li;
  const uint16_t* xr = x + (int64_t)min(m, M - 1) * K;
  const uint16_t* ar = a + (int64_t)min(j, r - 1) * K;
  const bool mv = m < M, jv = j < r;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = (K + 31) / 32;
  int c = wave;
  for (; c + WAVES < nsteps; c += 2 * WAVES) {
    const int k0 = 32 * c + 8 * lg, k1 = k0 + 32 * WAVES;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const uint4 x0 = mv ? ld16(xr + k0) : z, a0 = jv ? ld16(ar + k0) : z;
    const uint4 x1 = (mv && k1 < K) ? ld16(xr + k1) : z, a1 = (jv && k1 < K) ? ld16(ar + k1) : z;
    acc = mfma16x16x32(as_bf16x8(x0), as_bf16x8(a0), acc);
    acc = mfma16x16x32(as_bf16x8(x1), as_bf16x8(a1), acc);
  }
  for (; c < nsteps; c += WAVES) {
    const int k0 = 32 * c + 8 * lg;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const uint4 x0 = (mv && k0 < K) ? ld16(xr + k0) : z, a0 = (jv && k0 < K) ? ld16(ar + k0) : z;
    acc = mfma16x16x32(as_bf16x8(x0), as_bf16x8(a0), acc);
  }
  __shared__ f32x4 red[WAVES][kWave];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w][lane];
    // lane holds rows 4*lg + v (tokens), column li (rank index)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = m0 + 4 * lg + v, jj = j0 + li;
      if (mm < M && jj < r) t[(int64_t)mm * r + jj] = s * sum[v];
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny (decode) kernel.
//   grid.x: row groups of 16*NT output features; grid.y: token groups of 16*MT.
//   WAVES waves per workgroup split the 128-wide K chunks round-robin.
// ---------------------------------------------------------------------------
template <int MT, int NT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void skinny_kernel(
    const uint16_t* __restrict__ x, int M, int N, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, const float* __restrict__ t,
    const uint16_t* __restrict__ lb, int r, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT);
  const int m0 = blockIdx.y * (16 * MT);
  const bool k32 = (K & 31) == 0;  // code rows are 16-byte aligned
  const int64_t cst = K / 2, sst = K / 16;

  const uint8_t* crow[NT];
  const uint8_t* srow[NT];
  bool nv[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int n = n0 + 16 * i + li;
    nv[i] = n < N;
    crow[i] = codes + (int64_t)min(n, N - 1) * cst;
    srow[i] = scales + (int64_t)min(n, N - 1) * sst;
  }
  const uint16_t* xrow[MT];
  bool mv[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int m = m0 + 16 * j + li;
    mv[j] = m < M;
    xrow[j] = x + (int64_t)min(m, M - 1) * K;
  }

  f32x4 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunk = (K + 127) / 128;
  for (int c = wave; c < nchunk; c += WAVES) {
    const int kb = 128 * c + 32 * lg;  // first k of this lane's 32-wide slice
    const int kv = K - kb;             // valid k from kb: >= 32, 16, or <= 0
    uint32_t cw[NT][4];
    uint32_t sw[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      cw[i][0] = cw[i][1] = cw[i][2] = cw[i][3] = 0u;
      sw[i] = 0u;
      if (nv[i] && kv > 0) {
        const uint8_t* cp = crow[i] + kb / 2;
        const uint8_t* sp = srow[i] + kb / 16;
        if (kv >= 32 && k32) {
          const uint4 v = ld16(cp);
          cw[i][0] = v.x; cw[i][1] = v.y; cw[i][2] = v.z; cw[i][3] = v.w;
          sw[i] = *reinterpret_cast<const uint16_t*>(sp);
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(cp);
          cw[i][0] = v.x; cw[i][1] = v.y;
          sw[i] = sp[0];
          if (kv >= 32) {
            const uint2 u = *reinterpret_cast<const uint2*>(cp + 8);
            cw[i][2] = u.x; cw[i][3] = u.y;
            sw[i] |= (uint32_t)sp[1] << 8;
          }
        }
      }
    }
    float s0[NT], s1[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      s0[i] = e4m3_to_f32(sw[i] & 0xFFu);
      s1[i] = e4m3_to_f32(sw[i] >> 8);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 xv[MT];
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (mv[j] && 8 * s < kv) v = ld16(xrow[j] + kb + 8 * s);
        xv[j] = as_bf16x8(v);
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const bf16x8 a = dequant8(cw[i][s], s < 2 ? s0[i] : s1[i]);
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[i][j] = mfma16x16x32(a, xv[j], acc[i][j]);
      }
    }
  }

  const float st = *tensor_scale;
  const bool rvec = (r & 7) == 0;
  // Epilogue of one 16x16 tile: lane holds features n = n0+16i+4lg+v and token m = m0+16j+li.
  auto epilogue = [&](int i, int j, f32x4 v) {
    f32x4 lo = {0.f, 0.f, 0.f, 0.f};
    if (r > 0) {
      const int na = n0 + 16 * i + li;  // B row for the A operand
      const int mb = m0 + 16 * j + li;  // t row for the B operand
      for (int j0 = 0; j0 < r; j0 += 32) {
        const int jj = j0 + 8 * lg;
        uint4 bw = make_uint4(0, 0, 0, 0);
        float tv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (jj < r) {
          if (rvec) {
            if (na < N) bw = ld16(lb + (int64_t)na * r + jj);
            if (mb < M) {
              const float4 t0 = *reinterpret_cast<const float4*>(t + (int64_t)mb * r + jj);
              const float4 t1 = *reinterpret_cast<const float4*>(t + (int64_t)mb * r + jj + 4);
              tv[0] = t0.x; tv[1] = t0.y; tv[2] = t0.z; tv[3] = t0.w;
              tv[4] = t1.x; tv[5] = t1.y; tv[6] = t1.z; tv[7] = t1.w;
            }
          } else {
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const bool ok = jj + e < r;
              h[e] = (ok && na < N) ? lb[(int64_t)na * r + jj + e] : 0u;
              tv[e] = (ok && mb < M) ? t[(int64_t)mb * r + jj + e] : 0.f;
            }
            bw = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
          }
        }
        uint4 th, tl;
        split_bf16x8(tv, th, tl);
        lo = mfma16x16x32(as_bf16x8(bw), as_bf16x8(th), lo);
        lo = mfma16x16x32(as_bf16x8(bw), as_bf16x8(tl), lo);
      }
    }
    const int m = m0 + 16 * j + li;
    const int nf = n0 + 16 * i + 4 * lg;
    if (m < M) {
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(st * v[e] + lo[e]);
      uint16_t* yp = y + (int64_t)m * N + nf;
      if ((N & 3) == 0 && nf + 3 < N) {
        *reinterpret_cast<uint2*>(yp) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (nf + e < N) yp[e] = (uint16_t)o[e];
      }
    }
  };

  if constexpr (WAVES == 1) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j) epilogue(i, j, acc[i][j]);
  } else {
    __shared__ f32x4 red[WAVES][NT * MT][kWave];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j) red[wave][i * MT + j][lane] = acc[i][j];
    __syncthreads();
    for (int tl = wave; tl < NT * MT; tl += WAVES) {
      f32x4 sum = red[0][tl][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][tl][lane];
      epilogue(tl / MT, tl % MT, sum);
    }
  }
}

struct SkinnyCfg {
  int mt, nt, waves;
};

// Pick tile counts so that the launch has ~1.5k+ waves in flight (6 per CU)
// while the LDS reduction buffer stays within 64 KB (waves*nt*mt <= 64).
SkinnyCfg pick_skinny(int64_t m, int64_t n, int64_t k) {
  const int mt = m <= 16 ? 1 : m <= 32 ? 2 : m <= 64 ? 4 : 8;
  const int64_t gy = (m + 16 * mt - 1) / (16 * mt);
  const int64_t nchunk = (k + 127) / 128;
  SkinnyCfg best{mt, 2, 1};
  int64_t best_waves = -1;
  for (int nt : {4, 2}) {
    if (mt == 8 && nt == 4) continue;  // accumulators + operands would exceed the register file
    const int64_t groups = (n + 16 * nt - 1) / (16 * nt) * gy;
    int wmax = std::min<int64_t>(16, 64 / (nt * mt));
    wmax = (int)std::min<int64_t>(wmax, std::max<int64_t>(1, nchunk));
    int w = 1;
    while (w < wmax && groups * w < 1536) w *= 2;
    w = std::min(w, wmax);
    // round down to a power of two the templates provide
    int wp = 1;
    while (wp * 2 <= w) wp *= 2;
    const int64_t tot = groups * wp;
    if (tot >= 1536) return SkinnyCfg{mt, nt, wp};
    if (tot > best_waves) {
      best_waves = tot;
      best = SkinnyCfg{mt, nt, wp};
    }
  }
  return best;
}

template <int MT, int NT, int W>
hipError_t run_skinny(dim3 grid, hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes,
                      const uint8_t* scales, const float* ts, const float* t, const uint16_t* b, int r, uint16_t* y) {
  hipLaunchKernelGGL((skinny_kernel<MT, NT, W>), grid, dim3(W * kWave), 0, st, x, M, N, K, codes, scales, ts, t, b,
                     r, y);
  return hipGetLastError();
}

template <int MT, int NT>
hipError_t run_skinny_w(int w, dim3 grid, hipStream_t st, const uint16_t* x, int M, int N, int K,
                        const uint8_t* codes, const uint8_t* scales, const float* ts, const float* t,
                        const uint16_t* b, int r, uint16_t* y) {
  // only waves * MT * NT <= 64 is instantiated: the reduction buffer is at most 64 KB of LDS
#define FP4RL_CASE(W_)                                                                             \
  case W_:                                                                                         \
    if constexpr (W_ * MT * NT <= 64) return run_skinny<MT, NT, W_>(grid, st, x, M, N, K, codes, scales, ts, t, b, r, y); \
    break;
  switch (w) {
    FP4RL_CASE(1) FP4RL_CASE(2) FP4RL_CASE(4) FP4RL_CASE(8) FP4RL_CASE(16)
    default: break;
  }
#undef FP4RL_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* a, int64_t r, float lora_scale,
                            float* t, hipStream_t stream) {
  const dim3 grid((unsigned)((m + 15) / 16), (unsigned)((r + 15) / 16));
  if (m <= 256)
    hipLaunchKernelGGL(lora_down_kernel<16>, grid, dim3(16 * kWave), 0, stream, x, (int)m, (int)k, a, (int)r,
                       lora_scale, t);
  else
    hipLaunchKernelGGL(lora_down_kernel<4>, grid, dim3(4 * kWave), 0, stream, x, (int)m, (int)k, a, (int)r,
                       lora_scale, t);
  return hipGetLastError();
}

hipError_t launch_fp4_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                             const uint8_t* scales, const float* tensor_scale, const float* t, const uint16_t* b,
                             int64_t r, uint16_t* y, hipStream_t stream) {
  const SkinnyCfg cfg = pick_skinny(m, n, k);
  const dim3 grid((unsigned)((n + 16 * cfg.nt - 1) / (16 * cfg.nt)), (unsigned)((m + 16 * cfg.mt - 1) / (16 * cfg.mt)));
  const int M = (int)m, N = (int)n, K = (int)k, R = (int)r;
#define FP4RL_SKINNY(MT_, NT_) \
  if (cfg.mt == MT_ && cfg.nt == NT_) \
    return run_skinny_w<MT_, NT_>(cfg.waves, grid, stream, x, M, N, K, codes, scales, tensor_scale, t, b, R, y);
  FP4RL_SKINNY(1, 2) FP4RL_SKINNY(1, 4) FP4RL_SKINNY(2, 2) FP4RL_SKINNY(2, 4)
  FP4RL_SKINNY(4, 2) FP4RL_SKINNY(4, 4) FP4RL_SKINNY(8, 2)
#undef FP4RL_SKINNY
  return hipErrorInvalidValue;
}

}  // namespace fp4rl
