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
// (nibble + 1/16 scale byte). The weights come in the tiled NVFP4 layout
// (16-row x 128-k tiles, 1 KB of codes + 128 B of scales, stored in the order
// the MFMA lanes consume them), so every wave load is one contiguous 1 KB
// (one lane = 32 consecutive k of one row = two blocks). It dequantises in
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
// LoRA down-projection, split along K into `gridDim.z` slices of `kslice`:
//   part[z][m][j] = s * sum_{k in slice z} x[m][k] A[j][k].
// One workgroup per 16x16 tile of t and K slice; its waves take the 32-wide
// steps of the slice round-robin, U steps' loads at a time, and reduce
// through LDS. With one slice, `part` is t itself; otherwise the slices are
// summed in slice order by lora_reduce_kernel or by the linear's epilogue.
// ---------------------------------------------------------------------------
template <int WAVES, int U = 4>
__global__ __launch_bounds__(WAVES * kWave) void lora_down_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                   const uint16_t* __restrict__ a, int r, float s,
                                                                   int kslice, float* __restrict__ part) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.x * 16, j0 = blockIdx.y * 16;
  const int m = m0 + li, j = j0 + li;
  const uint16_t* xr = x + (int64_t)min(m, M - 1) * K;
  const uint16_t* ar = a + (int64_t)min(j, r - 1) * K;
  const bool mv = m < M, jv = j < r;
  const int kbeg = blockIdx.z * kslice;
  const int kend = min(K, kbeg + kslice);
  const int nsteps = (kend - kbeg + 31) / 32;
  const int mine = nsteps > wave ? (nsteps - wave + WAVES - 1) / WAVES : 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < mine; g0 += U) {
    uint4 xv[U], av[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = kbeg + 32 * (wave + WAVES * (g0 + u)) + 8 * lg;
      const bool kv = (g0 + u < mine) && k0 < kend;
      xv[u] = (mv && kv) ? ld16(xr + k0) : make_uint4(0, 0, 0, 0);
      av[u] = (jv && kv) ? ld16(ar + k0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = mfma16x16x32(as_bf16x8(xv[u]), as_bf16x8(av[u]), acc);
  }
  __shared__ f32x4 red[WAVES][kWave];
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w][lane];
    // lane holds rows 4*lg + v (tokens), column li (rank index)
    float* dst = part + (int64_t)blockIdx.z * M * r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = m0 + 4 * lg + v, jj = j0 + li;
      if (mm < M && jj < r) dst[(int64_t)mm * r + jj] = s * sum[v];
    }
  }
}

// t[i] = sum_{z < slices} part[z][i], summed in slice order (deterministic).
__global__ void lora_reduce_kernel(const float* __restrict__ part, int slices, int64_t count, float* __restrict__ t) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float acc = part[i];
  for (int z = 1; z < slices; ++z) acc += part[(int64_t)z * count + i];
  t[i] = acc;
}

// ---------------------------------------------------------------------------
// Skinny (decode) kernel.
//   grid.x: row groups of 16*NT output features; grid.y: token groups of 16*MT.
//   WAVES waves per workgroup split the 128-wide K chunks round-robin.
// ---------------------------------------------------------------------------
// U: chunks per pipeline group; with two groups in registers, one group's
// code + activation registers (U * (4 NT + 16 MT)) are kept near 64 per lane
// (32 for 1024-thread workgroups, whose waves have at most 128 registers).
constexpr int skinny_group(int mt, int nt, int waves) {
  const int budget = waves >= 16 ? 32 : 64;
  const int u = mt <= 4 ? budget / (4 * nt + 16 * mt) : 2;
  return u > 0 ? u : 1;
}
template <int MT, int NT, int WAVES, int U = skinny_group(MT, NT, WAVES)>
__global__ __launch_bounds__(WAVES * kWave) void skinny_kernel(
    const uint16_t* __restrict__ x, int M, int N, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, const float* __restrict__ t,
    int tks, const uint16_t* __restrict__ lb, int r, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * (16 * NT);
  const int m0 = blockIdx.y * (16 * MT);
  // Tiled weights: tile (rt, c) = 16 rows x 128 k; this lane's 16 code bytes
  // sit at 16 * lane and its 2 scale bytes at 2 * lane of the tile. Bases are
  // wave-uniform (scalar registers); lanes add 32-bit offsets. Row tiles past
  // the matrix are clamped to the last one (their rows are never stored).
  const int RT = (N + 15) >> 4, KC = (K + 127) >> 7;
  const int rt0 = blockIdx.x * NT;
  const uint8_t* cbase = codes + (int64_t)rt0 * KC * 1024;  // uniform
  const uint8_t* sbase = scales + (int64_t)rt0 * KC * 128;  // uniform
  const uint32_t clane = 16 * lane, slane = 2 * lane;
  int toff[NT];  // tile offset of row tile i, in tiles (uniform)
#pragma unroll
  for (int i = 0; i < NT; ++i) toff[i] = (min(rt0 + i, RT - 1) - rt0) * KC;
  // Activations: tokens past M are clamped to the last token (columns never stored).
  const uint16_t* xbase = x + (int64_t)m0 * K;  // uniform
  uint32_t xoff[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) xoff[j] = (uint32_t)(min(m0 + 16 * j + li, M - 1) - m0) * (uint32_t)K + 32 * lg;
  const bool kfull = (K & 127) == 0;  // every chunk holds 128 valid k

  f32x4 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each wave owns the 128-wide K chunks wave, wave+WAVES, ...; they are
  // processed in groups of U. Software pipeline with two register buffers:
  // the code, scale and (for MT <= 4) activation loads of group g+1 are in
  // flight while group g is dequantised and multiplied. With MT = 8 the
  // activation fragments of a chunk (128 registers) are loaded step by step.
  constexpr bool XPRE = MT <= 4;
  constexpr int XU = XPRE ? U : 1;
  const int nchunk = (K + 127) / 128;
  const int mine = nchunk > wave ? (nchunk - wave + WAVES - 1) / WAVES : 0;

  struct Group {
    uint32_t cw[U][NT][4];
    uint32_t sw[U][NT];
    uint4 xq[XU][4][MT];
  };
  auto load_group = [&](int g0, Group& G) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // chunks past this wave's share are clamped (loaded, never used)
      const int c = __builtin_amdgcn_readfirstlane(min(wave + WAVES * (g0 + u), nchunk - 1));
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const uint8_t* ct = cbase + (int64_t)(toff[i] + c) * 1024;  // uniform tile address
        const uint4 v = ld_nt16(ct + clane);
        G.cw[u][i][0] = v.x; G.cw[u][i][1] = v.y; G.cw[u][i][2] = v.z; G.cw[u][i][3] = v.w;
        const uint8_t* st = sbase + (int64_t)(toff[i] + c) * 128;
        G.sw[u][i] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(st + slane));
      }
      if constexpr (XPRE) {
        const uint16_t* xc = xbase + 128 * c;  // uniform
        if (kfull || c < nchunk - 1) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < MT; ++j) G.xq[u][s][j] = ld16(xc + xoff[j] + 8 * s);
        } else {  // last, partial chunk: k past K is not read
          const int kv = K - 128 * c - 32 * lg;
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < MT; ++j)
              G.xq[u][s][j] = 8 * s < kv ? ld16(xc + xoff[j] + 8 * s) : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto compute_group = [&](int g0, const Group& G) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u >= mine) break;  // uniform across the wave
      const int c = __builtin_amdgcn_readfirstlane(wave + WAVES * (g0 + u));
      const int kv = K - 128 * c - 32 * lg;
      const uint16_t* xc = xbase + 128 * c;
      float s0[NT], s1[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        s0[i] = __builtin_amdgcn_cvt_f32_fp8((int)G.sw[u][i], 0);  // OCP E4M3, exact
        s1[i] = __builtin_amdgcn_cvt_f32_fp8((int)G.sw[u][i], 1);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 xv[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          if constexpr (XPRE) {
            xv[j] = as_bf16x8(G.xq[u][s][j]);
          } else {
            xv[j] = as_bf16x8((kfull || 8 * s < kv) ? ld16(xc + xoff[j] + 8 * s) : make_uint4(0, 0, 0, 0));
          }
        }
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const bf16x8 a = dequant8(G.cw[u][i][s], s < 2 ? s0[i] : s1[i]);
#pragma unroll
          for (int j = 0; j < MT; ++j) acc[i][j] = mfma16x16x32(a, xv[j], acc[i][j]);
        }
      }
    }
  };
  Group ga, gb;
  if (mine > 0) load_group(0, ga);
  for (int g0 = 0; g0 < mine; g0 += 2 * U) {
    if (g0 + U < mine) load_group(g0 + U, gb);
    compute_group(g0, ga);
    if (g0 + U >= mine) break;
    if (g0 + 2 * U < mine) load_group(g0 + 2 * U, ga);
    compute_group(g0 + U, gb);
  }

  const float st = *tensor_scale;
  const bool rvec = (r & 7) == 0;
  const int64_t tstride = (int64_t)M * r;
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
              for (int q = 0; q < tks; ++q) {  // K-slices of t, summed in order
                const float* tp = t + (int64_t)q * tstride + (int64_t)mb * r + jj;
                const float4 t0 = *reinterpret_cast<const float4*>(tp);
                const float4 t1 = *reinterpret_cast<const float4*>(tp + 4);
                tv[0] += t0.x; tv[1] += t0.y; tv[2] += t0.z; tv[3] += t0.w;
                tv[4] += t1.x; tv[5] += t1.y; tv[6] += t1.z; tv[7] += t1.w;
              }
            }
          } else {
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const bool ok = jj + e < r;
              h[e] = (ok && na < N) ? lb[(int64_t)na * r + jj + e] : 0u;
              if (ok && mb < M)
                for (int q = 0; q < tks; ++q) tv[e] += t[(int64_t)q * tstride + (int64_t)mb * r + jj + e];
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

// ---------------------------------------------------------------------------
// GEMV kernel for one or two tokens (VALU, no MFMA).
//   One workgroup per 16-row weight tile; its WAVES waves take the 128-wide K
//   chunks round-robin, U chunks per software-pipeline group (two register
//   buffers). The tokens are staged once in LDS (all lanes of a lane group
//   read the same 64 bytes: LDS broadcast). Per 16-byte code piece a lane
//   converts 32 E2M1 codes to bf16 pairs with the hardware convert at unit
//   scale, accumulates each 16-element block with v_dot2_f32_bf16 and applies
//   the block's E4M3 scale once: ~1 VALU instruction per weight, half the
//   MFMA path's dequantisation cost. Lane groups and waves are reduced by
//   shuffles and LDS in a fixed order. The LoRA operands (B rows of the tile
//   and t, its K-slices summed in order) are staged in LDS before the main
//   loop so their load latency overlaps it.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int MTOK, int WAVES, int U>
__global__ __launch_bounds__(WAVES * kWave) void gemv_kernel(
    const uint16_t* __restrict__ x, int M, int N, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, const float* __restrict__ t,
    int tks, const uint16_t* __restrict__ lb, int r, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const int KC = (K + 127) >> 7, Kp = KC * 128;
  const int rt = blockIdx.x;
  const int nchunk = KC;
  const int mine = nchunk > wave ? (nchunk - wave + WAVES - 1) / WAVES : 0;
  const uint8_t* cbase = codes + (int64_t)rt * KC * 1024;
  const uint8_t* sbase = scales + (int64_t)rt * KC * 128;
  const uint32_t clane = 16 * lane, slane = 2 * lane;

  struct Group {
    uint32_t cw[U][4];
    uint32_t sw[U];
  };
  auto load_group = [&](int g0, Group& G) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = __builtin_amdgcn_readfirstlane(min(wave + WAVES * (g0 + u), nchunk - 1));
      const uint4 v = ld_nt16(cbase + (int64_t)c * 1024 + clane);
      G.cw[u][0] = v.x; G.cw[u][1] = v.y; G.cw[u][2] = v.z; G.cw[u][3] = v.w;
      G.sw[u] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sbase + (int64_t)c * 128 + slane));
    }
  };
  Group ga, gb;
  if (mine > 0) load_group(0, ga);  // weights first: the staging below overlaps their latency

  // LDS: tokens [MTOK][Kp] bf16 (zero past K and past M), t summed [MTOK][r], B rows [16][r], reduction
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* tsum = reinterpret_cast<float*>(smem + (size_t)MTOK * Kp * 2);
  float* bsh = tsum + MTOK * r;
  float* red = bsh + 16 * r;  // [WAVES][MTOK][16]
  const int pieces = MTOK * Kp / 8;
  for (int i = threadIdx.x; i < pieces; i += WAVES * kWave) {
    const int m = i / (Kp / 8), kk = (i - m * (Kp / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M && kk < K) v = ld16(x + (int64_t)m * K + kk);
    *reinterpret_cast<uint4*>(xs + m * Kp + kk) = v;
  }
  const int64_t tstride = (int64_t)M * r;
  for (int i = threadIdx.x; i < MTOK * r; i += WAVES * kWave) {
    const int m = i / r, j = i - m * r;
    float a = 0.0f;
    if (m < M)
      for (int q = 0; q < tks; ++q) a += t[q * tstride + (int64_t)m * r + j];  // slice order
    tsum[i] = a;
  }
  for (int i = threadIdx.x; i < 16 * r; i += WAVES * kWave) {
    const int row = i / r, j = i - row * r;
    const int n = 16 * rt + row;
    bsh[i] = n < N ? bf16_lo(lb[(int64_t)n * r + j]) : 0.0f;
  }
  __syncthreads();

  float acc[MTOK];
#pragma unroll
  for (int m = 0; m < MTOK; ++m) acc[m] = 0.0f;
  auto compute_group = [&](int g0, const Group& G) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u >= mine) break;  // uniform across the wave
      const int c = __builtin_amdgcn_readfirstlane(wave + WAVES * (g0 + u));
      uint4 xv[MTOK][4];
#pragma unroll
      for (int m = 0; m < MTOK; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xv[m][q] = *reinterpret_cast<const uint4*>(xs + m * Kp + 128 * c + 32 * lg + 8 * q);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const float sc = blk == 0 ? __builtin_amdgcn_cvt_f32_fp8((int)G.sw[u], 0)
                                  : __builtin_amdgcn_cvt_f32_fp8((int)G.sw[u], 1);
        float p[MTOK];
#pragma unroll
        for (int m = 0; m < MTOK; ++m) p[m] = 0.0f;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t w = G.cw[u][2 * blk + d];
          const bf16x2 g0v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
          const bf16x2 g1v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
          const bf16x2 g2v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
          const bf16x2 g3v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
#pragma unroll
          for (int m = 0; m < MTOK; ++m) {
            const uint4 xq = xv[m][2 * blk + d];  // x[k .. k+7] of this dword's 8 codes
            p[m] = __builtin_amdgcn_fdot2_f32_bf16(g0v, __builtin_bit_cast(bf16x2, xq.x), p[m], false);
            p[m] = __builtin_amdgcn_fdot2_f32_bf16(g1v, __builtin_bit_cast(bf16x2, xq.y), p[m], false);
            p[m] = __builtin_amdgcn_fdot2_f32_bf16(g2v, __builtin_bit_cast(bf16x2, xq.z), p[m], false);
            p[m] = __builtin_amdgcn_fdot2_f32_bf16(g3v, __builtin_bit_cast(bf16x2, xq.w), p[m], false);
          }
        }
#pragma unroll
        for (int m = 0; m < MTOK; ++m) acc[m] = fmaf(sc, p[m], acc[m]);
      }
    }
  };
  for (int g0 = 0; g0 < mine; g0 += 2 * U) {
    if (g0 + U < mine) load_group(g0 + U, gb);
    compute_group(g0, ga);
    if (g0 + U >= mine) break;
    if (g0 + 2 * U < mine) load_group(g0 + 2 * U, ga);
    compute_group(g0 + U, gb);
  }

  // the four lane groups hold partial sums of the same row: fold them, then the waves
#pragma unroll
  for (int m = 0; m < MTOK; ++m) {
    acc[m] += __shfl_xor(acc[m], 16, kWave);
    acc[m] += __shfl_xor(acc[m], 32, kWave);
  }
  if (lg == 0) {
#pragma unroll
    for (int m = 0; m < MTOK; ++m) red[(wave * MTOK + m) * 16 + li] = acc[m];
  }
  __syncthreads();
  if (threadIdx.x < 16 * MTOK) {
    const int row = threadIdx.x & 15, m = threadIdx.x >> 4;
    const int n = 16 * rt + row;
    if (m < M && n < N) {
      float sum = 0.0f;
      for (int w = 0; w < WAVES; ++w) sum += red[(w * MTOK + m) * 16 + row];
      float lo = 0.0f;
      for (int j = 0; j < r; ++j) lo = fmaf(tsum[m * r + j], bsh[row * r + j], lo);
      y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16(*tensor_scale * sum + lo);
    }
  }
}

size_t gemv_lds_bytes(int mtok, int64_t k, int64_t r, int waves) {
  const int64_t kp = (k + 127) / 128 * 128;
  return (size_t)(mtok * kp * 2 + (mtok * r + 16 * r) * 4 + waves * mtok * 16 * 4);
}

struct SkinnyCfg {
  int mt, nt, waves;
};

// Token tiles (16*mt) cover M; row tiles per workgroup (nt) grow with M so the
// activation fragments a lane loads are reused across more weight rows; the
// waves per workgroup split K so that ~4k waves are in flight (16 per CU),
// within a 64 KB LDS reduction buffer (waves * nt * mt <= 64).
SkinnyCfg pick_skinny(int64_t m, int64_t n, int64_t k) {
  const int mt = m <= 16 ? 1 : m <= 32 ? 2 : m <= 64 ? 4 : 8;
  const int nt = m <= 16 ? 1 : 2;
  const int64_t gy = (m + 16 * mt - 1) / (16 * mt);
  const int64_t groups = (n + 16 * nt - 1) / (16 * nt) * gy;
  const int64_t kc = (k + 127) / 128;
  const int wcap = mt == 1 ? 16 : 8;  // 1024-thread groups leave 128 registers per lane: MT = 1 only
  const int wmax = (int)std::min<int64_t>(std::min<int64_t>(wcap, 64 / (nt * mt)), std::max<int64_t>(1, kc));
  int w = 1;
  while (w * 2 <= wmax && groups * w < 4096) w *= 2;
  return SkinnyCfg{mt, nt, w};
}

template <int MT, int NT, int W>
hipError_t run_skinny(dim3 grid, hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes,
                      const uint8_t* scales, const float* ts, const float* t, int tks, const uint16_t* b, int r,
                      uint16_t* y) {
  hipLaunchKernelGGL((skinny_kernel<MT, NT, W>), grid, dim3(W * kWave), 0, st, x, M, N, K, codes, scales, ts, t, tks,
                     b, r, y);
  return hipGetLastError();
}

template <int MT, int NT>
hipError_t run_skinny_w(int w, dim3 grid, hipStream_t st, const uint16_t* x, int M, int N, int K,
                        const uint8_t* codes, const uint8_t* scales, const float* ts, const float* t, int tks,
                        const uint16_t* b, int r, uint16_t* y) {
  // only waves * MT * NT <= 64 is instantiated: the reduction buffer is at most 64 KB of LDS
#define FP4RL_CASE(W_)                                                                             \
  case W_:                                                                                         \
    if constexpr (W_ * MT * NT <= 64 && (W_ < 16 || MT == 1)) return run_skinny<MT, NT, W_>(grid, st, x, M, N, K, codes, scales, ts, t, tks, b, r, y); \
    break;
  switch (w) {
    FP4RL_CASE(1) FP4RL_CASE(2) FP4RL_CASE(4) FP4RL_CASE(8) FP4RL_CASE(16)
    default: break;
  }
#undef FP4RL_CASE
  return hipErrorInvalidValue;
}

}  // namespace

int lora_splits(int64_t m, int64_t k, int64_t r) {
  (void)r;
  if (m > 128) return 1;  // prefill: token tiles already fill the chip
  // The linear's epilogue re-reads every slice for its 16*mt tokens: keep
  // slices * mt <= 8 so that stays a few KB per workgroup.
  const int mt = m <= 16 ? 1 : m <= 32 ? 2 : m <= 64 ? 4 : 8;
  const int64_t by_k = std::max<int64_t>(1, k / 512);  // at least 512 k per slice
  return (int)std::min<int64_t>(8 / mt, by_k);
}

static int64_t slice_len(int64_t k, int splits) { return ((k + splits - 1) / splits + 31) / 32 * 32; }

hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* a, int64_t r, float lora_scale,
                            int splits, float* part, hipStream_t stream) {
  const int64_t ks = slice_len(k, splits);
  const dim3 grid((unsigned)((m + 15) / 16), (unsigned)((r + 15) / 16), (unsigned)((k + ks - 1) / ks));
  if ((m + 15) / 16 * ((r + 15) / 16) * grid.z <= 256)
    hipLaunchKernelGGL(lora_down_kernel<16>, grid, dim3(16 * kWave), 0, stream, x, (int)m, (int)k, a, (int)r,
                       lora_scale, (int)ks, part);
  else
    hipLaunchKernelGGL(lora_down_kernel<4>, grid, dim3(4 * kWave), 0, stream, x, (int)m, (int)k, a, (int)r,
                       lora_scale, (int)ks, part);
  return hipGetLastError();
}

int lora_slices(int64_t k, int splits) {
  const int64_t ks = slice_len(k, splits);
  return (int)((k + ks - 1) / ks);
}

hipError_t launch_lora_reduce(const float* part, int slices, int64_t count, float* t, hipStream_t stream) {
  hipLaunchKernelGGL(lora_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, part, slices,
                     count, t);
  return hipGetLastError();
}

// GEMV path: one or two tokens, when the staged tokens and LoRA operands fit
// in 64 KB of LDS.
static int gemv_waves(int64_t n, int64_t k) {
  const int64_t rt = (n + 15) / 16, kc = (k + 127) / 128;
  int w = 1;
  while (w < 16 && w < kc && rt * w < 8192) w *= 2;
  return w;
}

static bool use_gemv(int64_t m, int64_t n, int64_t k, int64_t r) {
  return m <= 2 && gemv_lds_bytes((int)m, k, r, gemv_waves(n, k)) <= 65536;
}

template <int MTOK, int W>
hipError_t run_gemv(hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes, const uint8_t* scales,
                    const float* ts, const float* t, int tks, const uint16_t* b, int r, uint16_t* y) {
  constexpr int U = W >= 16 ? 4 : 8;
  const size_t lds = gemv_lds_bytes(MTOK, K, r, W);
  hipLaunchKernelGGL((gemv_kernel<MTOK, W, U>), dim3((unsigned)((N + 15) / 16)), dim3(W * kWave), lds, st, x, M, N, K,
                     codes, scales, ts, t, tks, b, r, y);
  return hipGetLastError();
}

template <int MTOK>
hipError_t run_gemv_w(int w, hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes,
                      const uint8_t* scales, const float* ts, const float* t, int tks, const uint16_t* b, int r,
                      uint16_t* y) {
  switch (w) {
    case 1: return run_gemv<MTOK, 1>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y);
    case 2: return run_gemv<MTOK, 2>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y);
    case 4: return run_gemv<MTOK, 4>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y);
    case 8: return run_gemv<MTOK, 8>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y);
    case 16: return run_gemv<MTOK, 16>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y);
    default: return hipErrorInvalidValue;
  }
}

const char* fp4_linear_kernel_name(int64_t m, int64_t n, int64_t k, int64_t r) {
  static const char* const kNames[4][3][5] = {
#define FP4RL_NAME_ROW(MT_, NT_)                                                                           \
  {"skinny_kernel<" #MT_ ", " #NT_ ", 1>", "skinny_kernel<" #MT_ ", " #NT_ ", 2>",                          \
   "skinny_kernel<" #MT_ ", " #NT_ ", 4>", "skinny_kernel<" #MT_ ", " #NT_ ", 8>",                          \
   "skinny_kernel<" #MT_ ", " #NT_ ", 16>"}
      {FP4RL_NAME_ROW(1, 1), FP4RL_NAME_ROW(1, 2), FP4RL_NAME_ROW(1, 4)},
      {FP4RL_NAME_ROW(2, 1), FP4RL_NAME_ROW(2, 2), FP4RL_NAME_ROW(2, 4)},
      {FP4RL_NAME_ROW(4, 1), FP4RL_NAME_ROW(4, 2), FP4RL_NAME_ROW(4, 4)},
      {FP4RL_NAME_ROW(8, 1), FP4RL_NAME_ROW(8, 2), FP4RL_NAME_ROW(8, 4)},
#undef FP4RL_NAME_ROW
  };
  static const char* const kGemv[2][5] = {
      {"gemv_kernel<1, 1, 8>", "gemv_kernel<1, 2, 8>", "gemv_kernel<1, 4, 8>", "gemv_kernel<1, 8, 8>",
       "gemv_kernel<1, 16, 4>"},
      {"gemv_kernel<2, 1, 8>", "gemv_kernel<2, 2, 8>", "gemv_kernel<2, 4, 8>", "gemv_kernel<2, 8, 8>",
       "gemv_kernel<2, 16, 4>"}};
  if (use_gemv(m, n, k, r)) {
    int wi = 0;
    while ((1 << wi) < gemv_waves(n, k)) ++wi;
    return kGemv[m - 1][wi];
  }
  const SkinnyCfg c = pick_skinny(m, n, k);
  const int mi = c.mt == 1 ? 0 : c.mt == 2 ? 1 : c.mt == 4 ? 2 : 3;
  const int ni = c.nt == 1 ? 0 : c.nt == 2 ? 1 : 2;
  int wi = 0;
  while ((1 << wi) < c.waves) ++wi;
  return kNames[mi][ni][wi];
}

hipError_t launch_fp4_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                             const uint8_t* scales, const float* tensor_scale, const float* t, int tks,
                             const uint16_t* b, int64_t r, uint16_t* y, hipStream_t stream) {
  const int M = (int)m, N = (int)n, K = (int)k, R = (int)r;
  if (use_gemv(m, n, k, r)) {
    const int w = gemv_waves(n, k);
    return m == 1 ? run_gemv_w<1>(w, stream, x, M, N, K, codes, scales, tensor_scale, t, tks, b, R, y)
                  : run_gemv_w<2>(w, stream, x, M, N, K, codes, scales, tensor_scale, t, tks, b, R, y);
  }
  const SkinnyCfg cfg = pick_skinny(m, n, k);
  const dim3 grid((unsigned)((n + 16 * cfg.nt - 1) / (16 * cfg.nt)), (unsigned)((m + 16 * cfg.mt - 1) / (16 * cfg.mt)));
#define FP4RL_SKINNY(MT_, NT_) \
  if (cfg.mt == MT_ && cfg.nt == NT_) \
    return run_skinny_w<MT_, NT_>(cfg.waves, grid, stream, x, M, N, K, codes, scales, tensor_scale, t, tks, b, R, y);
  FP4RL_SKINNY(1, 1) FP4RL_SKINNY(2, 2) FP4RL_SKINNY(4, 2) FP4RL_SKINNY(8, 2)
#undef FP4RL_SKINNY
  return hipErrorInvalidValue;
}

}  // namespace fp4rl
