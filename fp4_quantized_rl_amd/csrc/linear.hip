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
// (one lane = 32 k of one row, four groups of 8). It dequantises in
// registers (hardware E2M1 convert at unit scale, times the E4M3 block
// scale: exact in bf16) and feeds v_mfma_f32_16x16x32_bf16 with the weights
// as the 16-row A operand and up to 8 tiles of 16 tokens as B operands. The
// K dimension is split across the waves of a workgroup and reduced through
// LDS (deterministic, no atomics); the LoRA up-projection runs in the
// epilogue as extra MFMA steps, with t split into bf16 hi + lo parts.
//
// Within one MFMA the order of the 32 k values is free as long as A and B
// use the same one. Step j (0..3) of a 128-wide chunk takes k = 32 j .. 32 j
// + 31: lane group g = lane/16 supplies k = 32 j + 8 g .. + 7, which is word j
// of the lane's 16-byte code load. On the activation side the four lane
// groups of one token then read 64 consecutive bytes per load instruction.
#include <algorithm>
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace fp4rl {
namespace {

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Buffer descriptor word 3 for raw (untyped) 32-bit element access on gfx950.
constexpr int kBufferWord3 = 0x00020000;
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
// Cache policy of agent-coherent loads: SC1 (the bits the compiler gives an
// agent-scope atomic load), so data stored by another XCD is seen.
constexpr int kCoherent = 16;
__device__ __forceinline__ f32x4 ld_coherent16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, kCoherent));
}
__device__ __forceinline__ float ld_coherent4(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0, kCoherent));
}
__device__ __forceinline__ void st_coherent16(f32x4 v, __amdgpu_buffer_rsrc_t rs, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v), rs, byte_off, 0, kCoherent);
}
__device__ __forceinline__ void st_coherent4(float v, __amdgpu_buffer_rsrc_t rs, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, byte_off, 0, kCoherent);
}

// Calls f(I, J) for every (I, J) < (TI, TJ) with compile-time indices, so that
// register arrays indexed by them never fall back to scratch memory (a plain
// loop over a large inlined body may be left rolled).
template <int TI, int TJ, int E = 0, class F>
__device__ __forceinline__ void for_tiles(F&& f) {
  if constexpr (E < TI * TJ) {
    f(std::integral_constant<int, E / TJ>{}, std::integral_constant<int, E % TJ>{});
    for_tiles<TI, TJ, E + 1>(f);
  }
}

// The four E4M3 scale bytes of a tiled scale word, decoded exactly (OCP e4m3fn).
__device__ __forceinline__ void scale4(uint32_t w, float (&sc)[4]) {
  sc[0] = __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
  sc[1] = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  sc[2] = __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
  sc[3] = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}

// One 16x16 tile of t (tokens m0.., ranks j0..) for K slice z, by WAVES
// waves; red: WAVES x 64 f32x4 of LDS. COHERENT stores are agent-scope
// atomics, for readers in the same launch on another XCD.
template <int WAVES, bool COHERENT, int U = 4>
__device__ __forceinline__ void lora_tile(const uint16_t* __restrict__ x, int M, int K,
                                          const uint16_t* __restrict__ a, int r, float s, int kslice, int m0, int j0,
                                          int z, f32x4* red, float* __restrict__ part) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int m = m0 + li, j = j0 + li;
  const uint16_t* xr = x + (int64_t)min(m, M - 1) * K;
  const uint16_t* ar = a + (int64_t)min(j, r - 1) * K;
  const bool mv = m < M, jv = j < r;
  const int kbeg = z * kslice;
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
  red[wave * kWave + lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = red[lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w * kWave + lane];
    // lane holds rows 4*lg + v (tokens), column li (rank index)
    float* dst = part + (int64_t)z * M * r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = m0 + 4 * lg + v, jj = j0 + li;
      if (mm < M && jj < r) {
        if constexpr (COHERENT)
          __hip_atomic_store(dst + (int64_t)mm * r + jj, s * sum[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          dst[(int64_t)mm * r + jj] = s * sum[v];
      }
    }
  }
}

// All RTN 16-rank tiles of t for TT 16-token tiles (m0..) and K slice z, by
// WAVES waves taking the 32-wide steps round-robin: each activation fragment
// is loaded once and feeds RTN MFMAs, each adapter fragment TT (ranks past r
// and tokens past M clamped, never stored); red: WAVES x TT x RTN x 64 f32x4
// of LDS, reduced in wave order.
template <int WAVES, int TT, int RTN, int U>
__device__ __forceinline__ void lora_rows(const uint16_t* __restrict__ x, int M, int K, const uint16_t* __restrict__ a,
                                          int r, float s, int kslice, int m0, int z, f32x4* red,
                                          float* __restrict__ part) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const uint16_t* xr[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) xr[u] = x + (int64_t)min(m0 + 16 * u + li, M - 1) * K;
  const uint16_t* ar[RTN];
#pragma unroll
  for (int t = 0; t < RTN; ++t) ar[t] = a + (int64_t)min(16 * t + li, r - 1) * K;
  const int kbeg = z * kslice;
  const int kend = min(K, kbeg + kslice);
  const int nsteps = (kend - kbeg + 31) / 32;
  const int mine = nsteps > wave ? (nsteps - wave + WAVES - 1) / WAVES : 0;
  f32x4 acc[TT][RTN];
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int t = 0; t < RTN; ++t) acc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < mine; g0 += U) {
    uint4 xv[U][TT], av[U][RTN];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int k0 = kbeg + 32 * (wave + WAVES * (g0 + q)) + 8 * lg;
      const bool kv = (g0 + q < mine) && k0 < kend;
#pragma unroll
      for (int u = 0; u < TT; ++u) xv[q][u] = kv ? ld16(xr[u] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < RTN; ++t) av[q][t] = kv ? ld16(ar[t] + k0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
#pragma unroll
      for (int u = 0; u < TT; ++u)
#pragma unroll
        for (int t = 0; t < RTN; ++t) acc[u][t] = mfma16x16x32(as_bf16x8(xv[q][u]), as_bf16x8(av[q][t]), acc[u][t]);
  }
#pragma unroll
  for (int u = 0; u < TT; ++u)
#pragma unroll
    for (int t = 0; t < RTN; ++t) red[((wave * TT + u) * RTN + t) * kWave + lane] = acc[u][t];
  __syncthreads();
  float* dst = part + (int64_t)z * M * r;
  for (int e = wave; e < TT * RTN; e += WAVES) {
    const int u = e / RTN, t = e - u * RTN;
    f32x4 sum = red[e * kWave + lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[(w * TT * RTN + e) * kWave + lane];
    // lane holds rows 4*lg + v (tokens), column li (rank index)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = m0 + 16 * u + 4 * lg + v, jj = 16 * t + li;
      if (mm < M && jj < r) dst[(int64_t)mm * r + jj] = s * sum[v];
    }
  }
}

template <int WAVES, int TT, int RTN, int U>
__global__ __launch_bounds__(WAVES * kWave) void lora_down_rows_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                        const uint16_t* __restrict__ a, int r, float s,
                                                                        int kslice, float* __restrict__ part) {
  __shared__ f32x4 red[WAVES * TT * RTN * kWave];
  lora_rows<WAVES, TT, RTN, U>(x, M, K, a, r, s, kslice, blockIdx.x * 16 * TT, blockIdx.z, red, part);
}

// ---------------------------------------------------------------------------
// LoRA down-projection, split along K into `gridDim.z` slices of `kslice`:
//   part[z][m][j] = s * sum_{k in slice z} x[m][k] A[j][k].
// One workgroup per 16x16 tile of t and K slice; its waves take the 32-wide
// steps of the slice round-robin, U steps' loads at a time, and reduce
// through LDS. With one slice, `part` is t itself; otherwise the slices are
// summed in slice order by lora_reduce_kernel or by the linear's epilogue.
// ---------------------------------------------------------------------------
template <int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void lora_down_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                   const uint16_t* __restrict__ a, int r, float s,
                                                                   int kslice, float* __restrict__ part) {
  __shared__ f32x4 red[WAVES * kWave];
  lora_tile<WAVES, false>(x, M, K, a, r, s, kslice, blockIdx.x * 16, blockIdx.y * 16, blockIdx.z, red, part);
}

// Fused producers and the consumers' side of the handshake (LoraFuse).
// `flag`: one word of LDS.
template <int WAVES>
__device__ __forceinline__ void lora_produce(const LoraFuse& L, int pid, const uint16_t* __restrict__ x, int M, int K,
                                             int r, f32x4* red, uint32_t* flag) {
  const int ntile = L.mtiles * L.rtiles;
  if (pid >= ntile * L.slices) return;  // padding of the producer count to a multiple of 8
  const int z = pid / ntile, tile = pid - z * ntile;
  const int m0 = 16 * (tile % L.mtiles), j0 = 16 * (tile / L.mtiles);
  lora_tile<WAVES, true>(x, M, K, L.a, r, L.s, L.kslice, m0, j0, z, red, L.part);
  __builtin_amdgcn_s_waitcnt(0);  // this lane's stores of its slice are complete
  __syncthreads();
  if (L.slices > 1) {
    if (threadIdx.x == 0)
      *flag = __hip_atomic_fetch_add(L.tctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (uint32_t)L.slices - 1;
    __syncthreads();
    if (*flag == 0u) return;
    // the tile's last slice: t = part[0] + ... + part[slices-1], added in
    // slice order, into part[0]
    // (all slices' loads in flight at once: slices <= 8, and the t region,
    // slices * M * r floats, is far below 2^31 bytes)
    const int zbytes = 4 * M * r;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(L.part, 0, L.slices * zbytes, kBufferWord3);
    for (int e = threadIdx.x; e < 256; e += WAVES * kWave) {
      const int mm = m0 + (e >> 4), jj = j0 + (e & 15);
      if (mm < M && jj < r) {
        const int off = 4 * (mm * r + jj);
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = ld_coherent4(prs, min(q, L.slices - 1) * zbytes + off);
        float acc = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q < L.slices) acc += v[q];
        st_coherent4(acc, prs, off);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(L.tctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // this tile of t is complete; the workgroup that completes the last one
  // raises every group's ready flag
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(L.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)ntile - 1;
  __syncthreads();
  if (*flag != 0u) {
    if (threadIdx.x == 0) __hip_atomic_store(L.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((int)threadIdx.x < L.groups && L.withhold == 0u)
      __hip_atomic_store(L.lines + kLoraLineWords * threadIdx.x, L.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Consumers' side, for the workgroup that writes output tile `tile` of y
// (thread 0 does the memory accesses). It reads its group's ready flag early
// (lora_poll), so the latency overlaps other work; lora_wait then returns at
// once if it holds this call's epoch, else polls (bounded: a producer that
// never raises the flag leaves the error bit in the workspace, never a
// hang). Right after its wait the consumer counts itself on its group's line
// (lora_release) and, once its epilogue is issued, the group's last consumer
// clears the line (lora_reset_if_last), so every launch (a graph replay too)
// starts from cleared flags. The epoch covers what clearing cannot: when all
// of a group's consumers gave up, a flag its producer raises afterwards holds
// that call's epoch and never releases a later call early.
__device__ __forceinline__ uint32_t* lora_line(const LoraFuse& L, int tile) {
  return L.lines + kLoraLineWords * (tile % L.groups);
}

__device__ __forceinline__ uint32_t lora_poll(const LoraFuse& L, int tile) {
  return (L.producers > 0 && threadIdx.x == 0)
             ? __hip_atomic_load(lora_line(L, tile), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
             : 0u;
}

__device__ __forceinline__ void lora_wait(const LoraFuse& L, int tile, uint32_t seen) {
  if (L.producers > 0 && threadIdx.x == 0) {
    const uint32_t* f = lora_line(L, tile);
    for (uint32_t it = 0; seen != L.epoch && it < L.spin; ++it) {
      __builtin_amdgcn_s_sleep(8);
      seen = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (seen != L.epoch)
      __hip_atomic_fetch_or(L.err, kLinearErrLoraWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t lora_release(const LoraFuse& L, int tile) {
  return (L.producers > 0 && threadIdx.x == 0)
             ? __hip_atomic_fetch_add(lora_line(L, tile) + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
             : 0u;
}

__device__ __forceinline__ void lora_reset_if_last(const LoraFuse& L, int tile, uint32_t released_before) {
  if (L.producers > 0 && threadIdx.x == 0) {
    const int g = tile % L.groups;
    const int members = L.consumers / L.groups + (g < L.consumers % L.groups ? 1 : 0);
    if (released_before == (uint32_t)members - 1) {
      uint32_t* f = lora_line(L, tile);
      __hip_atomic_store(f, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(f + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// Epilogue of one 16x16 output tile held in MFMA D layout (lane = 16 g + i
// holds features nb + 4 g + v, v = 0..3, of token mb + i):
//   y = bf16(s_t * v + t B^T), t summed over its `tks` K-slices in slice order.
// The LoRA product runs as MFMA steps over r in 32-wide pieces: B rows of the
// tile are the A operand, t rows the B operand, t split into bf16 hi + lo.
// ---------------------------------------------------------------------------
// COH: t was written by other workgroups of this launch, so it is read with
// agent-coherent loads (16 bytes at a time, through a buffer descriptor).
// KB: K-slices of t loaded at once.
// rs: per-row scales (FP8 weights) in place of st, when set.
template <bool COH = false, int KB = 4>
__device__ __forceinline__ void store_tile(f32x4 v, int nb, int mb, int lane, int M, int N, float st,
                                           const float* __restrict__ t, int tks, const uint16_t* __restrict__ lb,
                                           int r, uint16_t* __restrict__ y, const float* __restrict__ rs = nullptr) {
  const int li = lane & 15, lg = lane >> 4;
  f32x4 lo = {0.f, 0.f, 0.f, 0.f};
  if (r > 0) {
    // (unused, and removed by the compiler, unless COH)
    const __amdgpu_buffer_rsrc_t trs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(t), 0, (int)(4 * (int64_t)tks * M * r), kBufferWord3);
    const bool rvec = (r & 7) == 0;
    const int64_t tstride = (int64_t)M * r;
    const int na = nb + li;  // B row for the A operand
    const int ma = mb + li;  // t row for the B operand
    for (int j0 = 0; j0 < r; j0 += 32) {
      const int jj = j0 + 8 * lg;
      uint4 bw = make_uint4(0, 0, 0, 0);
      float tv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (jj < r) {
        if (rvec) {
          if (na < N) bw = ld16(lb + (int64_t)na * r + jj);
          if (ma < M) {
            // K-slices of t, summed in order; a batch's loads are all in
            // flight at once (the last slice stands in for missing ones)
            const int64_t o0 = (int64_t)ma * r + jj;
            if constexpr (COH) {  // one slice (the producers added them)
              const f32x4 p0 = ld_coherent16(trs, (int)(4 * o0)), p1 = ld_coherent16(trs, (int)(4 * o0) + 16);
#pragma unroll
              for (int e = 0; e < 4; ++e) tv[e] += p0[e], tv[e + 4] += p1[e];
            } else if (tks == 1) {
              const f32x4* tp = reinterpret_cast<const f32x4*>(t + o0);
              const f32x4 p0 = tp[0], p1 = tp[1];
#pragma unroll
              for (int e = 0; e < 4; ++e) tv[e] += p0[e], tv[e + 4] += p1[e];
            } else {
              for (int q0 = 0; q0 < tks; q0 += KB) {
                f32x4 p[KB][2];
#pragma unroll
                for (int u = 0; u < KB; ++u) {
                  const f32x4* tp = reinterpret_cast<const f32x4*>(t + (int64_t)min(q0 + u, tks - 1) * tstride + o0);
                  p[u][0] = tp[0];
                  p[u][1] = tp[1];
                }
#pragma unroll
                for (int u = 0; u < KB; ++u)
                  if (q0 + u < tks) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) tv[e] += p[u][0][e], tv[e + 4] += p[u][1][e];
                  }
              }
            }
          }
        } else {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool ok = jj + e < r;
            h[e] = (ok && na < N) ? lb[(int64_t)na * r + jj + e] : 0u;
            if (ok && ma < M)
              for (int q = 0; q < tks; ++q) {
                const int64_t o = (int64_t)q * tstride + (int64_t)ma * r + jj + e;
                if constexpr (COH)
                  tv[e] += ld_coherent4(trs, (int)(4 * o));
                else
                  tv[e] += t[o];
              }
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
  const int m = mb + li;
  const int nf = nb + 4 * lg;
  if (m < M) {
    f32x4 sv = {st, st, st, st};
    if (rs != nullptr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[e] = rs[min(nf + e, N - 1)];
    }
    const uint32_t o01 = pack_bf16x2(sv[0] * v[0] + lo[0], sv[1] * v[1] + lo[1]);
    const uint32_t o23 = pack_bf16x2(sv[2] * v[2] + lo[2], sv[3] * v[3] + lo[3]);
    uint16_t* yp = y + (int64_t)m * N + nf;
    if ((N & 3) == 0 && nf + 3 < N) {
      *reinterpret_cast<uint2*>(yp) = make_uint2(o01, o23);
    } else {
      const uint32_t o[4] = {o01 & 0xFFFFu, o01 >> 16, o23 & 0xFFFFu, o23 >> 16};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (nf + e < N) yp[e] = (uint16_t)o[e];
    }
  }
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
    int tks, const uint16_t* __restrict__ lb, int r, uint16_t* __restrict__ y, LoraFuse lf) {
  __shared__ f32x4 red[WAVES][NT * MT][kWave];  // the waves' sums; fused LoRA producers use its first WAVES KB
  __shared__ uint32_t pflag;
  if ((int)blockIdx.x < lf.producers) {  // fused LoRA down-projection (grid.y is 1 then)
    lora_produce<WAVES>(lf, blockIdx.x, x, M, K, r, &red[0][0][0], &pflag);
    return;
  }
  const int bx = blockIdx.x - lf.producers;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int li = lane & 15, lg = lane >> 4;
  const int n0 = bx * (16 * NT);
  const int m0 = blockIdx.y * (16 * MT);
  // Tiled weights: tile (rt, c) = 16 rows x 128 k; this lane's 16 code bytes
  // sit at 16 * lane of the tile and its scale word (byte j = the block of
  // step j) at 4 * (16 (g / 2) + i). Bases are wave-uniform (scalar
  // registers); lanes add 32-bit offsets. Row tiles past the matrix are
  // clamped to the last one (their rows are never stored).
  const int RT = (N + 15) >> 4, KC = (K + 127) >> 7;
  const int rt0 = bx * NT;
  const uint8_t* cbase = codes + (int64_t)rt0 * KC * 1024;  // uniform
  const uint8_t* sbase = scales + (int64_t)rt0 * KC * 128;  // uniform
  const uint32_t clane = 16 * lane, slane = 4 * (16 * (lg >> 1) + li);
  int toff[NT];  // tile offset of row tile i, in tiles (uniform)
#pragma unroll
  for (int i = 0; i < NT; ++i) toff[i] = (min(rt0 + i, RT - 1) - rt0) * KC;
  // Activations: tokens past M are clamped to the last token (columns never stored).
  const uint16_t* xbase = x + (int64_t)m0 * K;  // uniform
  // the same rows through a buffer descriptor (32-bit byte offsets: the host keeps 2 M K below 2^31)
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xbase), 0, (int)(2u * (uint32_t)(min(M - m0, 16 * MT)) * (uint32_t)K), kBufferWord3);
  uint32_t xoff[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) xoff[j] = (uint32_t)(min(m0 + 16 * j + li, M - 1) - m0) * (uint32_t)K + 8 * lg;
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
        G.sw[u][i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(st + slane));
      }
      if constexpr (XPRE) {
        // pieces past K get an offset beyond the buffer and read as zero (no
        // per-lane branch: the compiler then waits for exactly the loads
        // each use needs)
        const int kv = K - 128 * c - 8 * lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t kout = 32 * s < kv ? 0u : 0x80000000u;
#pragma unroll
          for (int j = 0; j < MT; ++j)
            G.xq[u][s][j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)((2u * (xoff[j] + 128u * c + 32u * s)) | kout),
                                                             0, 0));
        }
      }
    }
  };
  auto compute_group = [&](int g0, const Group& G) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (g0 + u >= mine) break;  // uniform across the wave
      const int c = __builtin_amdgcn_readfirstlane(wave + WAVES * (g0 + u));
      const int kv = K - 128 * c - 8 * lg;
      const uint16_t* xc = xbase + 128 * c;
      float sc[NT][4];
#pragma unroll
      for (int i = 0; i < NT; ++i) scale4(G.sw[u][i], sc[i]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 xv[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          if constexpr (XPRE) {
            xv[j] = as_bf16x8(G.xq[u][s][j]);
          } else {
            xv[j] = as_bf16x8((kfull || 32 * s < kv) ? ld16(xc + xoff[j] + 32 * s) : make_uint4(0, 0, 0, 0));
          }
        }
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const bf16x8 a = dequant8(G.cw[u][i][s], sc[i][s]);
#pragma unroll
          for (int j = 0; j < MT; ++j) acc[i][j] = mfma16x16x32(a, xv[j], acc[i][j]);
        }
      }
    }
  };
  // Two groups in flight. In the steady state every load is issued
  // unconditionally (a group past this wave's chunks loads clamped chunks),
  // so the compiler waits for exactly the loads a group uses, never for the
  // group in flight; the last one or two groups run after the loop.
  Group ga, gb;
  load_group(0, ga);
  // (the scheduling barriers keep a group's loads together at its start:
  // sunk into the previous group's arithmetic they would each be waited on
  // at once)
  int g0 = 0;
  for (; g0 + 2 * U < mine; g0 += 2 * U) {
    load_group(g0 + U, gb);
    __builtin_amdgcn_sched_barrier(0);
    compute_group(g0, ga);
    load_group(g0 + 2 * U, ga);
    __builtin_amdgcn_sched_barrier(0);
    compute_group(g0 + U, gb);
  }
  if (g0 + U < mine) {
    load_group(g0 + U, gb);
    __builtin_amdgcn_sched_barrier(0);
    compute_group(g0, ga);
    compute_group(g0 + U, gb);
  } else {
    compute_group(g0, ga);
  }

  const float st = *tensor_scale;
  auto epilogue = [&](int i, int j, f32x4 v) {
    if (lf.producers > 0)
      store_tile<true>(v, n0 + 16 * i, m0 + 16 * j, lane, M, N, st, t, tks, lb, r, y);
    else
      store_tile<false, (WAVES >= 16 ? 1 : 4)>(v, n0 + 16 * i, m0 + 16 * j, lane, M, N, st, t, tks, lb, r, y);
  };
  const int ytile = blockIdx.y * (gridDim.x - lf.producers) + bx;  // fused LoRA group
  const uint32_t t_seen = lora_poll(lf, ytile);

  if constexpr (WAVES == 1) {
    lora_wait(lf, ytile, t_seen);
    const uint32_t released = lora_release(lf, ytile);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j) epilogue(i, j, acc[i][j]);
    lora_reset_if_last(lf, ytile, released);
  } else {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < MT; ++j) red[wave][i * MT + j][lane] = acc[i][j];
    __syncthreads();
    lora_wait(lf, ytile, t_seen);
    const uint32_t released = lora_release(lf, ytile);
    for (int tl = wave; tl < NT * MT; tl += WAVES) {
      f32x4 sum = red[0][tl][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][tl][lane];
      epilogue(tl / MT, tl % MT, sum);
    }
    lora_reset_if_last(lf, ytile, released);
  }
}

// ---------------------------------------------------------------------------
// Split-K MFMA kernel for 16 < M <= 128 tokens.
//   grid.x: groups of TM row tiles (16 TM output features); grid.y: groups of
//   TN token tiles; grid.z: ranges of `cpz` 128-wide K chunks. The W waves of
//   a workgroup take the chunks of its range round-robin and each covers all
//   TM x TN output tiles, so one activation fragment feeds TM MFMAs and one
//   weight fragment TN.
//   Activations pass through a private LDS slab per wave. The L1 merges the
//   addresses of consecutive lanes only, and the MFMA operand layout puts
//   consecutive lanes on different tokens (different rows of x); so a chunk
//   is loaded with 16 lanes per token row (contiguous 256 B), written to LDS
//   and read back in operand layout (rows padded to 272 B: conflict-free).
//   The waves' sums are reduced through LDS in wave order. With one K range
//   the workgroup stores y; otherwise it writes its fp32 partial tile to
//   part[z], and the last workgroup of the tile to arrive (a per-tile counter
//   in the workspace) adds the partials in z order, stores y and clears the
//   counter, so results do not depend on arrival order and the counters are
//   zero again when the kernel ends.
// ---------------------------------------------------------------------------
constexpr int kXRow = 136;  // bf16 per LDS token row: 128 + 8 of padding

// F8: the weights are E4M3 bytes [N][K] row-major with one fp32 scale per row
// (`scales` then points to N floats): a lane loads the 32 contiguous bytes
// k = 32 g .. + 31 of its row per chunk and step st takes k = 32 g + 8 st
// .. + 7 (the same order on the activation side, so the sum is the plain
// one); converted exactly to bf16, no block scale. With tok_scale set, x
// holds the tokens' E4M3 codes widened to bf16 (exact) and the sums are
// multiplied by each token's scale (W8A8). With one K range the
// workgroup stores y = bf16(s_n sum + t B^T), t (tks K-slices) made by a
// separate down-projection launch; otherwise it writes its K range's partial
// tile, times the row scales, to part[z] (plain stores; a later launch adds
// the ranges and the LoRA term). No counters and no fused producers.
template <int TM, int TN, int W, int D, bool F8 = false>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(D == 2 ? (TM <= 2 ? 4 : (F8 ? 2 : 3)) : 1))) void splitk_kernel(
    const uint16_t* __restrict__ x, int M, int N, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, const float* __restrict__ t, int tks,
    const uint16_t* __restrict__ lb, int r, uint16_t* __restrict__ y, int cpz, int nsplit, float* __restrict__ part,
    uint32_t* __restrict__ counters, LoraFuse lf, const float* __restrict__ tok_scale = nullptr) {
  static_assert(TM <= 4, "the reduction reuses the activation slabs: TM * TN KB <= TN * 4.25 KB");
  constexpr int TOK = 16 * TN;
  __shared__ __align__(16) uint16_t xs[W][TOK * kXRow];
  __shared__ uint32_t last_flag;
  if ((int)blockIdx.x < lf.producers) {  // fused LoRA down-projection
    lora_produce<W>(lf, blockIdx.x, x, M, K, r, reinterpret_cast<f32x4*>(&xs[0][0]), &last_flag);
    return;
  }
  const unsigned bid = blockIdx.x - lf.producers;  // producers are a multiple of 8: the XCD order holds
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const int RT = (N + 15) >> 4, KC = (K + 127) >> 7;
  // XCD-aware order of a 1-D grid: workgroups are dealt to the 8 XCDs in
  // turn, so workgroup L runs on XCD L % 8. All token groups and K ranges of
  // a row group get consecutive slots of one XCD: its weights are fetched
  // into that XCD's L2 once, and its partial sums stay there.
  const int GX = (RT + TM - 1) / TM, GT = (M + TOK - 1) / TOK;
  const int inner = (int)(bid >> 3) % (GT * nsplit);
  const int rg = (int)((bid >> 3) / (GT * nsplit)) * 8 + (int)(bid & 7);
  if (rg >= GX) return;  // padding of the row-group count to a multiple of 8
  const int tg = inner % GT, kz = inner / GT;
  const int rt0 = rg * TM, n0 = 16 * rt0, m0 = tg * TOK;
  const int cbeg = kz * cpz, cend = min(KC, cbeg + cpz);
  const int nch = max(0, cend - cbeg);
  const int mine = nch > wave ? (nch - wave + W - 1) / W : 0;

  const uint8_t* cbase = codes + (int64_t)rt0 * KC * 1024;  // uniform
  const uint8_t* sbase = scales + (int64_t)rt0 * KC * 128;
  const uint32_t clane = 16 * lane, slane = 4 * (16 * (lg >> 1) + li);
  int toff[TM];  // row tiles past the matrix are clamped to the last (never stored)
#pragma unroll
  for (int i = 0; i < TM; ++i) toff[i] = (min(rt0 + i, RT - 1) - rt0) * KC;
  const uint8_t* wrow[TM];  // F8: row n0 + 16 i + li (clamped), bytes from k = 32 g
#pragma unroll
  for (int i = 0; i < TM; ++i) wrow[i] = codes + (int64_t)min(n0 + 16 * i + li, N - 1) * K + 32 * lg;
  // Coalesced activation load: instruction q covers token rows 4 q + lg, 16 B
  // per lane, at a wave-uniform chunk base plus a 32-bit lane offset. Tokens
  // past M are clamped to the last one (their outputs are never stored).
  uint32_t xoff[TN * 4];  // bytes
#pragma unroll
  for (int q = 0; q < TN * 4; ++q) xoff[q] = 2u * ((uint32_t)min(m0 + 4 * q + lg, M - 1) * (uint32_t)K + 8 * li);
  uint16_t* slab = xs[wave];

  struct WStage {
    uint32_t cw[TM][F8 ? 8 : 4];
    uint32_t sw[TM];
  };
  struct XStage {
    uint4 v[TN * 4];
  };
  auto chunk_of = [&](int q) { return __builtin_amdgcn_readfirstlane(cbeg + wave + W * q); };
  auto load_w = [&](int q, WStage& S) {
    const int c = chunk_of(q);
    if constexpr (F8) {
      // K % 16 == 0: a 16-byte piece is all in or out of the row
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool in = 128 * c + 32 * lg + 16 * h < K;
          const uint4 v = in ? ld_nt16(wrow[i] + 128 * (int64_t)c + 16 * h) : make_uint4(0u, 0u, 0u, 0u);
          S.cw[i][4 * h] = v.x; S.cw[i][4 * h + 1] = v.y; S.cw[i][4 * h + 2] = v.z; S.cw[i][4 * h + 3] = v.w;
        }
      return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      // streaming loads: a row group's token groups follow each other on one XCD and find the tiles in L2
      const uint4 v = ld_nt16(cbase + (int64_t)(toff[i] + c) * 1024 + clane);
      S.cw[i][0] = v.x; S.cw[i][1] = v.y; S.cw[i][2] = v.z; S.cw[i][3] = v.w;
      S.sw[i] = *reinterpret_cast<const uint32_t*>(sbase + (int64_t)(toff[i] + c) * 128 + slane);
    }
  };
  auto load_x = [&](int q, XStage& S) {
    const int c = chunk_of(q);
    const uint8_t* xc = reinterpret_cast<const uint8_t*>(x + 128 * c);  // uniform
    if (c < KC - 1 || (K & 127) == 0) {
#pragma unroll
      for (int j = 0; j < TN * 4; ++j) S.v[j] = ld16(xc + xoff[j]);
    } else {  // the last, partial chunk: pieces past K read as zero (K % 16 == 0: a piece is all in or out)
      const bool kin = 128 * c + 8 * li < K;
#pragma unroll
      for (int j = 0; j < TN * 4; ++j) S.v[j] = kin ? ld16(xc + xoff[j]) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](const XStage& S) {
#pragma unroll
    for (int q = 0; q < TN * 4; ++q) *reinterpret_cast<uint4*>(slab + (4 * q + lg) * kXRow + 8 * li) = S.v[q];
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const WStage& S) {
    if constexpr (F8) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 xv[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          xv[j] = as_bf16x8(*reinterpret_cast<const uint4*>(slab + (16 * j + li) * kXRow + 32 * lg + 8 * st));
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          uint32_t o[4];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const uint32_t wd = S.cw[i][2 * st + d];
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd, true);
            o[2 * d] = pack_hi16(lo.x, lo.y);
            o[2 * d + 1] = pack_hi16(hi.x, hi.y);
          }
          const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(a, xv[j], acc[i][j]);
        }
      }
      return;
    }
    float sc[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i) scale4(S.sw[i], sc[i]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 xv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        xv[j] = as_bf16x8(*reinterpret_cast<const uint4*>(slab + (16 * j + li) * kXRow + 32 * st + 8 * lg));
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const bf16x8 a = dequant8(S.cw[i][st], sc[i][st]);
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(a, xv[j], acc[i][j]);
      }
    }
  };

  // Pipeline: a ring of D weight stages (D chunks of weights in flight) and
  // XS activation stages in registers while the current chunk is in LDS.
  // D = 3 with two activation stages covers HBM latency at one wave per
  // SIMD (shapes with few workgroups); D = 2 with one activation stage
  // needs few enough registers for three waves per SIMD, which hide each
  // other's latency when the grid has more than one workgroup per CU. The
  // ring is unrolled so every stage lives in fixed registers. The slab is
  // rewritten only after this wave's reads of it were issued (LDS operations
  // of one wave complete in order).
  static_assert(D == 2 || D == 3, "two or three weight stages");
  constexpr int XS = D - 1, UNR = D * XS;  // unrolled by lcm(D, XS) so both rings use fixed registers
  WStage ws[D];
  XStage xr[XS];  // activations of chunks q + 1 .. q + XS in flight while chunk q is computed
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < mine) load_w(u, ws[u]);
#pragma unroll
  for (int u = 0; u < XS; ++u)
    if (u < mine) load_x(u, xr[u]);
  for (int q0 = 0; q0 < mine; q0 += UNR) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int q = q0 + u;
      if (q >= mine) break;  // uniform across the wave
      store_x(xr[u % XS]);
      if (q + XS < mine) load_x(q + XS, xr[u % XS]);
      compute(ws[u % D]);
      if (q + D < mine) load_w(q + D, ws[u % D]);
    }
  }

  // Reduce the waves' sums: wave w's tiles go to its own slab, then tile e is
  // summed over the waves, in wave order, by wave e % W.
  const int ytile = tg * GX + rg;  // this workgroup's output tile (its K-split counter, its LoRA group)
  const uint32_t t_seen = nsplit == 1 ? lora_poll(lf, ytile) : 0u;  // fused LoRA: read early, checked below
  float* red = reinterpret_cast<float*>(slab);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) *reinterpret_cast<f32x4*>(red + ((i * TN + j) * kWave + lane) * 4) = acc[i][j];
  __syncthreads();
  const float st = F8 ? 1.0f : *tensor_scale;
  constexpr int NTILE = TM * TN;
  f32x4 sums[(NTILE + W - 1) / W];
#pragma unroll
  for (int e0 = 0; e0 < (NTILE + W - 1) / W; ++e0) {
    const int e = wave + W * e0;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    if (e < NTILE) {
#pragma unroll
      for (int w = 0; w < W; ++w)
        sum += *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(xs[w]) + (e * kWave + lane) * 4);
    }
    sums[e0] = sum;
  }
  if constexpr (F8) {
    const float* rs = reinterpret_cast<const float*>(scales);
    if (tok_scale != nullptr) {  // W8A8: the tokens are E4M3 codes, times their per-token scale
#pragma unroll
      for (int e0 = 0; e0 < (NTILE + W - 1) / W; ++e0) {
        const int e = wave + W * e0;
        if (e < NTILE) sums[e0] *= tok_scale[min(m0 + 16 * (e % TN) + li, M - 1)];
      }
    }
    if (nsplit == 1) {  // one K range: y = bf16(s_n sum + t B^T) here, t from the separate down-projection
#pragma unroll
      for (int e0 = 0; e0 < (NTILE + W - 1) / W; ++e0) {
        const int e = wave + W * e0;
        if (e < NTILE)
          store_tile(sums[e0], n0 + 16 * (e / TN), m0 + 16 * (e % TN), lane, M, N, 1.0f, t, tks, lb, r, y, rs);
      }
      return;
    }
    // part[kz][m][n] = s_n * (this K range's sum)
    float* pz = part + (int64_t)kz * M * N;
#pragma unroll
    for (int e0 = 0; e0 < (NTILE + W - 1) / W; ++e0) {
      const int e = wave + W * e0;
      if (e < NTILE) {
        const int m = m0 + 16 * (e % TN) + li, nf = n0 + 16 * (e / TN) + 4 * lg;
        if (m < M) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (nf + v < N) pz[(int64_t)m * N + nf + v] = rs[nf + v] * sums[e0][v];
        }
      }
    }
    return;
  }
  if (nsplit == 1) {
    lora_wait(lf, ytile, t_seen);
    const uint32_t released = lora_release(lf, ytile);
#pragma unroll
    for (int e0 = 0; e0 < (NTILE + W - 1) / W; ++e0) {
      const int e = wave + W * e0;
      if (e < NTILE) {
        if (lf.producers > 0)
          store_tile<true>(sums[e0], n0 + 16 * (e / TN), m0 + 16 * (e % TN), lane, M, N, st, t, tks, lb, r, y);
        else
          store_tile(sums[e0], n0 + 16 * (e / TN), m0 + 16 * (e % TN), lane, M, N, st, t, tks, lb, r, y);
      }
    }
    lora_reset_if_last(lf, ytile, released);
    return;
  }
  // K split over workgroups: publish this range's partial tile. The partials
  // and the counter are agent-scope atomic accesses (coherent across the
  // chip's L2 slices without flushing them); every lane waits for its stores
  // to complete before the workgroup barrier, and the counter is bumped only
  // after that barrier, so a workgroup that sees the last count sees every
  // partial.
  // Partials are addressed through a buffer descriptor (byte offsets; the
  // host keeps all nsplit * M * N of them below 2^31 bytes) so that 16-byte
  // accesses can carry the agent-coherent cache policy.
  const int zbytes = 4 * M * N;
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(part, 0, nsplit * zbytes, kBufferWord3);
  const bool nvec = (N & 3) == 0;  // rows of 16-byte aligned groups of four
#pragma unroll
  for (int e0 = 0; e0 < (NTILE + W - 1) / W; ++e0) {
    const int e = wave + W * e0;
    if (e < NTILE) {
      const int m = m0 + 16 * (e % TN) + li, nf = n0 + 16 * (e / TN) + 4 * lg;
      if (m < M) {
        const int off = kz * zbytes + 4 * (m * N + nf);
        if (nvec) {
          if (nf < N) st_coherent16(sums[e0], prs, off);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (nf + v < N) st_coherent4(sums[e0][v], prs, off + 4 * v);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this lane's stores are complete
  __syncthreads();
  uint32_t* ctr = counters + ytile;
  uint32_t t_seen2 = 0u;
  if (threadIdx.x == 0) {
    t_seen2 = lora_poll(lf, ytile);  // in flight together with the tile count
    const uint32_t before = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = before == (uint32_t)nsplit - 1 ? 1u : 0u;
  }
  __syncthreads();
  if (last_flag == 0u) return;
  lora_wait(lf, ytile, t_seen2);
  const uint32_t released = lora_release(lf, ytile);
#pragma unroll
  for (int e0 = 0; e0 < (NTILE + W - 1) / W; ++e0) {
    const int e = wave + W * e0;
    if (e < NTILE) {
      const int m = m0 + 16 * (e % TN) + li, nf = n0 + 16 * (e / TN) + 4 * lg;
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
      if (m < M) {
        // all of a batch's loads in flight at once, added in split order
        // (results do not depend on arrival); elements past N are summed but
        // never stored, and reads past the buffer return zero
        const int off = 4 * (m * N + nf);
        constexpr int kB = 8;
        for (int z0 = 0; z0 < nsplit; z0 += kB) {
          f32x4 pz[kB];
#pragma unroll
          for (int u = 0; u < kB; ++u) {
            const int zo = min(z0 + u, nsplit - 1) * zbytes + off;
            if (nvec) {
              pz[u] = ld_coherent16(prs, zo);
            } else {
#pragma unroll
              for (int v = 0; v < 4; ++v) pz[u][v] = ld_coherent4(prs, zo + 4 * v);
            }
          }
#pragma unroll
          for (int u = 0; u < kB; ++u)
            if (z0 + u < nsplit) sum += pz[u];
        }
      }
      if (lf.producers > 0)
        store_tile<true>(sum, n0 + 16 * (e / TN), m0 + 16 * (e % TN), lane, M, N, st, t, tks, lb, r, y);
      else
        store_tile(sum, n0 + 16 * (e / TN), m0 + 16 * (e % TN), lane, M, N, st, t, tks, lb, r, y);
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lora_reset_if_last(lf, ytile, released);
}

// ---------------------------------------------------------------------------
// Mid-batch kernel for 96 < M <= 128 tokens on wide matrices: every weight
// tile is fetched and dequantised for all the tokens at once.
//   A workgroup computes 32 RW WR output features x 32 TGW WT tokens with
//   W = WR WT waves: wave (wr, wt) owns RW groups of 32 features and TGW
//   groups of 32 tokens, and runs the 32x32x16 bf16 MFMA with dequantised
//   weights as the A operand and activations as the B operand, so a weight
//   fragment feeds TGW MFMAs and an activation fragment read from LDS feeds
//   RW. Eight waves (two per SIMD) let one wave's dequantisation and loads
//   overlap another's MFMAs; a single wave per SIMD runs them one after the
//   other (measured: loads and staging, MFMA and dequantisation added up).
//   The waves share the activations: a chunk of 128 k for all the
//   workgroup's tokens is loaded by the whole workgroup (16 lanes per token
//   row) two chunks ahead, stored in one of two LDS slabs (rows padded to
//   272 B: conflict-free fragment reads) and read by every wave; one barrier
//   per chunk. Weights stream through a ring of D register stages per wave.
//   MFMA slots: a lane (row r = lane % 32, half h = lane / 32) loads lane
//   positions (r % 16, 2h) and (r % 16, 2h + 1) of its row's tile (16 bytes
//   each, both under the block scales of p = h); step (j, q) of a chunk
//   takes word j of position 2h + q, i.e. k = 32 j + 16 h + 8 q .. + 7, and
//   the activation fragment of the same lane holds the same k. A lane's
//   result holds token lane % 32 of its group and features 8 b + 4 h + e.
//   The LoRA update runs after the contraction as further MFMA steps over r
//   (B rows as the A operand, t split into bf16 hi + lo as the B operand),
//   added to the s_t-scaled sums. One workgroup per row group covers all of
//   K: the kernel serves matrices wide enough to give every CU one.
//   Measured limit (32B gate at 128 tokens, 40 chunks per workgroup, about
//   1.2 us each): loads, activation staging and the barrier take 0.7 us a
//   chunk on their own (each workgroup pulls 32 KB of activations and 18 KB
//   of weights through its CU's vector cache per chunk), MFMA and
//   dequantisation add the rest; they overlap little because the barrier
//   keeps the waves in step.
// ---------------------------------------------------------------------------
template <int RW, int TGW, int WR, int WT, int D>
__global__ __launch_bounds__(WR * WT * kWave) void mid_kernel(
    const uint16_t* __restrict__ x, int M, int N, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, const float* __restrict__ t, int tks,
    const uint16_t* __restrict__ lb, int r, uint16_t* __restrict__ y, LoraFuse lf, int nsplit = 1, int cps = 0,
    float* __restrict__ part = nullptr) {
  constexpr int W = WR * WT;
  constexpr int TOK = 32 * TGW * WT;  // tokens of the workgroup
  constexpr int ROWS = 32 * RW * WR;  // features of the workgroup
  constexpr int SLAB = TOK * kXRow;   // bf16 per activation slab
  __shared__ __align__(16) uint16_t xs[2 * SLAB];
  __shared__ uint32_t last_flag;
  static_assert(2 * SLAB * 2 >= W * kWave * 16, "the LoRA producers' reduction fits in the slabs");
  if ((int)blockIdx.x < lf.producers) {  // fused LoRA down-projection
    lora_produce<W>(lf, blockIdx.x, x, M, K, r, reinterpret_cast<f32x4*>(xs), &last_flag);
    return;
  }
  // row group (the producers come first); with part set, K range z of it:
  // chunks cbeg .. cbeg + cps - 1
  const int L = (int)blockIdx.x - lf.producers;
  const int rg = part != nullptr ? L / nsplit : L;
  const int z = part != nullptr ? L - rg * nsplit : 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wr = wave % WR, wt = wave / WR;
  const int lr = lane & 31, lh = lane >> 5;
  const int RT = (N + 15) >> 4, KC = (K + 127) >> 7;
  const int nw = ROWS * rg + 32 * RW * wr;  // this wave's features nw + 32 i + 0 .. 31, i < RW
  const int mw = 32 * TGW * wt;             // this wave's tokens mw + 32 g + 0 .. 31, g < TGW
  const int cbeg = part != nullptr ? z * cps : 0;
  const int nch = part != nullptr ? min(KC - cbeg, cps) : KC;  // chunks of 128 k

  // weights: tile of row nw + 32 i + lr (clamped: rows past N are computed, never stored)
  const uint8_t* cl[RW];
  const uint8_t* sl[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int tile = min(((nw + 32 * i) >> 4) + (lr >> 4), RT - 1);
    cl[i] = codes + (int64_t)tile * KC * 1024 + 16 * (32 * lh + (lr & 15));
    sl[i] = scales + (int64_t)tile * KC * 128 + 64 * lh + 4 * (lr & 15);
  }
  // Every load below is unconditional (chunk indices past K are clamped to
  // the last chunk, and their data is never used): with no
  // branches around the loads, the compiler waits only for the ones a step
  // consumes, so the prefetched chunks stay in flight across the loop.
  struct WStage {
    uint4 c0[RW], c1[RW];
    uint32_t s[RW];
  };
  auto load_w = [&](int q, WStage& S) {
    const int64_t c = cbeg + min(q, nch - 1);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      S.c0[i] = ld_nt16(cl[i] + c * 1024);
      S.c1[i] = ld_nt16(cl[i] + c * 1024 + 256);
      S.s[i] = *reinterpret_cast<const uint32_t*>(sl[i] + c * 128);
    }
  };
  // activations: piece p = tid + 64 W u of the chunk is token row p / 16, k = 8 (p % 16) .. + 7,
  // read through a buffer descriptor over x: pieces past K take an offset past
  // the buffer, which reads as zero (K % 16 == 0: a piece is all in or out)
  constexpr int XP = TOK * 16 / (W * kWave);  // pieces per thread
  static_assert(XP * W * kWave == TOK * 16, "whole pieces per thread");
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, 2 * M * K, kBufferWord3);
  uint32_t xoff[XP];  // bytes (tokens past M clamped to the last)
#pragma unroll
  for (int u = 0; u < XP; ++u) {
    const int p = (int)threadIdx.x + W * kWave * u;
    xoff[u] = 2u * ((uint32_t)min(p >> 4, M - 1) * (uint32_t)K + 8u * (uint32_t)(p & 15));
  }
  const int kcol = 8 * ((int)threadIdx.x & 15);  // the same k offset for every piece of this thread
  auto load_x = [&](int q, uint4 (&v)[XP]) {
    const int c = cbeg + min(q, nch - 1);
    const uint32_t base = 256u * (uint32_t)c, past = 128 * c + kcol < K ? 0u : 0x80000000u;
#pragma unroll
    for (int u = 0; u < XP; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)((xoff[u] + base) | past), 0, 0));
  };
  auto store_x = [&](int slab, const uint4 (&v)[XP]) {
#pragma unroll
    for (int u = 0; u < XP; ++u) {
      const int p = (int)threadIdx.x + W * kWave * u;
      *reinterpret_cast<uint4*>(xs + slab * SLAB + (p >> 4) * kXRow + 8 * (p & 15)) = v[u];
    }
  };

  f32x16 acc[RW][TGW];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int g = 0; g < TGW; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  auto compute = [&](int slab, const WStage& S) {
    float sc[RW][4];
#pragma unroll
    for (int i = 0; i < RW; ++i) scale4(S.s[i], sc[i]);
    const uint16_t* xb = xs + slab * SLAB + (mw + lr) * kXRow + 16 * lh;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        bf16x8 b[TGW];
#pragma unroll
        for (int g = 0; g < TGW; ++g)
          b[g] = as_bf16x8(*reinterpret_cast<const uint4*>(xb + g * 32 * kXRow + 32 * j + 8 * q));
#pragma unroll
        for (int i = 0; i < RW; ++i) {
          const uint4& cw = q == 0 ? S.c0[i] : S.c1[i];
          const uint32_t word = j == 0 ? cw.x : j == 1 ? cw.y : j == 2 ? cw.z : cw.w;
          const bf16x8 a = dequant8(word, sc[i][j]);
#pragma unroll
          for (int g = 0; g < TGW; ++g) acc[i][g] = mfma32x32x16(a, b[g], acc[i][g]);
        }
      }
  };

  // Pipeline: weight stages for chunks q + 1 .. q + D - 1 and activation
  // stages for chunks q + 1 .. q + XS in registers while chunk q is
  // computed; chunk q + 1's activations go to the other slab after the
  // compute (the barrier that ended chunk q - 1 guarantees that no wave
  // still reads it). The prologue issues its loads in the loop's order, so
  // the loop entry and its back edge see the same loads in flight. A range
  // of fewer chunks loads its last chunk again in their place (clamped,
  // unused).
  static_assert(D >= 2 && D <= 4, "two to four weight stages");
  constexpr int XS = 3;                      // activation chunks in flight
  constexpr int UNR = 12;                    // a multiple of D, XS and 2: every stage in fixed registers; the loads drain once per body (loop entry)
  static_assert(UNR % D == 0 && UNR % XS == 0 && UNR % 2 == 0, "whole rings per unrolled body");
  WStage ws[D];
  uint4 xr[XS][XP];
  if (nch > 0) {  // uniform across the workgroup
    load_x(0, xr[0]);
#pragma unroll
    for (int u = 0; u < XS - 1; ++u) {
      load_x(u + 1, xr[u + 1]);
      if (u < D) load_w(u, ws[u]);
    }
#pragma unroll
    for (int u = XS - 1; u < D; ++u) load_w(u, ws[u]);
    store_x(0, xr[0]);
    load_x(XS, xr[0]);
  }
  __syncthreads();
  for (int q0 = 0; q0 < nch; q0 += UNR) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int q = q0 + u;
      if (q >= nch) break;  // uniform across the workgroup
      // the next chunk's activations go to the other slab first (the
      // barrier that ended chunk q - 1 guarantees that no wave still reads
      // it) and a later chunk's activation loads are issued, so they are in
      // flight during the compute of chunk q; the weight stage that chunk q
      // used is refilled after it
      store_x((u + 1) & 1, xr[(u + 1) % XS]);
      load_x(q + 1 + XS, xr[(u + 1) % XS]);
      compute(u & 1, ws[u % D]);
      load_w(q + D, ws[u % D]);
      __syncthreads();
    }
  }

  if (part != nullptr) {  // K range z: s_t times its sums as fp32 partials (a later launch adds them)
    const float st = *tensor_scale;
    float* pz = part + (int64_t)z * M * N;
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int g = 0; g < TGW; ++g) {
        const int m = mw + 32 * g + lr;
        if (m >= M) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int nf = nw + 32 * i + 8 * b + 4 * lh;
          const f32x4 v = {st * acc[i][g][4 * b], st * acc[i][g][4 * b + 1], st * acc[i][g][4 * b + 2],
                           st * acc[i][g][4 * b + 3]};
          float* pp = pz + (int64_t)m * N + nf;
          if ((N & 3) == 0 && nf + 3 < N) {
            *reinterpret_cast<f32x4*>(pp) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (nf + e < N) pp[e] = v[e];
          }
        }
      }
    return;
  }
  const uint32_t t_seen = lora_poll(lf, rg);  // fused LoRA: read early, checked below
  const float st = *tensor_scale;
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int g = 0; g < TGW; ++g) acc[i][g] *= st;
  uint32_t released = 0u;
  if (r > 0) {
    lora_wait(lf, rg, t_seen);
    released = lora_release(lf, rg);
    // y += t B^T: 16 ranks per step, lane (r, h) takes ranks 16 s + 8 h .. + 7
    const bool coh = lf.producers > 0;  // t written by this launch's producers: agent-coherent loads
    const __amdgpu_buffer_rsrc_t trs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(t), 0, (int)(4 * (int64_t)tks * M * r), kBufferWord3);
    const int64_t tstride = (int64_t)M * r;
    for (int j0 = 0; j0 < r; j0 += 16) {
      const int jj = j0 + 8 * lh;
      uint4 th[TGW], tl[TGW];
#pragma unroll
      for (int g = 0; g < TGW; ++g) {
        const int ma = min(mw + 32 * g + lr, M - 1);
        float tv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (coh && (r & 3) == 0) {  // 16-byte loads: (ma r + jj) is a multiple of 4
          const int o = 4 * (ma * r + jj);
          if (jj < r) {
            const f32x4 v = ld_coherent16(trs, o);
            tv[0] = v[0]; tv[1] = v[1]; tv[2] = v[2]; tv[3] = v[3];
          }
          if (jj + 4 < r) {
            const f32x4 v = ld_coherent16(trs, o + 16);
            tv[4] = v[0]; tv[5] = v[1]; tv[6] = v[2]; tv[7] = v[3];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (jj + e < r) {
              const int64_t o = (int64_t)ma * r + jj + e;
              if (coh) {
                tv[e] = ld_coherent4(trs, (int)(4 * o));
              } else {
                for (int z = 0; z < tks; ++z) tv[e] += t[(int64_t)z * tstride + o];
              }
            }
          }
        }
        split_bf16x8(tv, th[g], tl[g]);
      }
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int na = min(nw + 32 * i + lr, N - 1);
        uint4 bw = make_uint4(0, 0, 0, 0);
        if (jj < r) {
          if ((r & 7) == 0) {
            bw = ld16(lb + (int64_t)na * r + jj);
          } else {
            uint32_t hv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = jj + e < r ? lb[(int64_t)na * r + jj + e] : 0u;
            bw = make_uint4(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16));
          }
        }
#pragma unroll
        for (int g = 0; g < TGW; ++g) {
          acc[i][g] = mfma32x32x16(as_bf16x8(bw), as_bf16x8(th[g]), acc[i][g]);
          acc[i][g] = mfma32x32x16(as_bf16x8(bw), as_bf16x8(tl[g]), acc[i][g]);
        }
      }
    }
  }

  // lane holds token mw + 32 g + lr, features nw + 32 i + 8 b + 4 lh + e (register 4 b + e)
  auto store_y = [&](int i, int g, const f32x16& v) {
    const int m = mw + 32 * g + lr;
    if (m >= M) return;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int nf = nw + 32 * i + 8 * b + 4 * lh;
      uint16_t* yp = y + (int64_t)m * N + nf;
      const uint32_t o01 = pack_bf16x2(v[4 * b], v[4 * b + 1]), o23 = pack_bf16x2(v[4 * b + 2], v[4 * b + 3]);
      if ((N & 3) == 0 && nf + 3 < N) {
        *reinterpret_cast<uint2*>(yp) = make_uint2(o01, o23);
      } else {
        const uint32_t o[4] = {o01 & 0xFFFFu, o01 >> 16, o23 & 0xFFFFu, o23 >> 16};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (nf + e < N) yp[e] = (uint16_t)o[e];
      }
    }
  };

#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int g = 0; g < TGW; ++g) store_y(i, g, acc[i][g]);
  if (r > 0) lora_reset_if_last(lf, rg, released);
}

// ---------------------------------------------------------------------------
// Prefill GEMM (M > 128 tokens): a workgroup computes 64 WAVES output
// features x 128 tokens over all of K with WAVES waves (4 or 8); wave w owns
// features 64 w .. +63 (two 32-row tiles, the 32x32x16 MFMA with dequantised
// weights as A) against all four 32-token groups, so each dequantised
// fragment feeds four MFMAs.
//   Activations go from HBM straight into LDS (buffer loads with an LDS
//   destination: no staging registers, no LDS store instructions), in the
//   MFMA operand order: one 1 KB fragment per (token group, 16-k step), lane
//   l's 16 bytes at 16 l, so every operand read is one conflict-free
//   contiguous 1 KB. Two slabs of 32 fragments (64 KB): chunk q + 1 loads
//   into one while chunk q is read from the other; one barrier per chunk.
//   Weights go to registers one chunk ahead.
//   With 64 KB of LDS and at most 256 registers per lane, a CU holds two
//   waves per SIMD: two four-wave workgroups (the barrier and load waits of
//   one overlap the MFMAs of the other) or one eight-wave workgroup, whose
//   512 features share each activation chunk (68 KB of loads per chunk
//   instead of 100 KB for the same flops on the CU).
//   Within a chunk the fragments of the next 16-k step (four LDS reads, two
//   dequantisations) are prepared while the current step's eight MFMAs run.
//   Grid order is XCD-aware: the 8 XCDs take workgroups in turn, and each
//   XCD works through super-tiles of 8 row groups x 4 token groups, so the
//   workgroups that run together on one XCD share their weights and
//   activations in its L2.
// ---------------------------------------------------------------------------
constexpr int kPfTok = 128;
typedef __attribute__((address_space(3))) void* lds_ptr;

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(
    const uint16_t* __restrict__ x, int M, int N, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, const float* __restrict__ t, int tks,
    const uint16_t* __restrict__ lb, int r, uint16_t* __restrict__ y) {
  constexpr int RW = 2, TG = 4, ROWS = 32 * RW * WAVES;
  static_assert((WAVES == 4 || WAVES == 8) && 32 * TG == kPfTok, "tile shape");
  constexpr int NFRAG = TG * 8;       // 1 KB activation fragments per chunk: (g, j, q)
  constexpr int FPW = NFRAG / WAVES;  // fragments loaded per wave
  __shared__ __align__(1024) uint8_t xs[2][NFRAG * 1024];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lr = lane & 31, lh = lane >> 5;
  const int RT = (N + 15) >> 4, KC = (K + 127) >> 7;
  const int GR = (N + ROWS - 1) / ROWS, GT = (M + kPfTok - 1) / kPfTok;
  // workgroup -> (row group, token group): XCD = L % 8; slot j = L / 8 of that
  // XCD; super-tile s = 8 (j / 32) + XCD covers row groups 8 sr .. +7 and
  // token groups 4 stt .. +3, its 32 tiles taken row group fastest
  const int L = blockIdx.x, xcd = L & 7, j = L >> 3;
  const int s = 8 * (j >> 5) + xcd, within = j & 31;
  const int nstt = (GT + 3) / 4;
  const int sr = s / nstt, stt = s - sr * nstt;
  const int rg = 8 * sr + (within & 7), tg = 4 * stt + (within >> 3);
  if (rg >= GR || tg >= GT) return;
  const int m0 = tg * kPfTok;
  const int nw = rg * ROWS + 32 * RW * wave;  // this wave's features nw + 32 i + 0 .. 31

  // weights: lane (lr, lh) takes row nw + 32 i + lr (rows past N clamped to
  // the last tile: computed, never stored); in chunk step (j, q) its word j
  // of c_q holds k = 32 j + 16 lh + 8 q .. + 7, block 2 j + lh of its scales
  const uint8_t* cl[RW];
  const uint8_t* sl[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int tile = min(((nw + 32 * i) >> 4) + (lr >> 4), RT - 1);
    cl[i] = codes + (int64_t)tile * KC * 1024 + 16 * (32 * lh + (lr & 15));
    sl[i] = scales + (int64_t)tile * KC * 128 + 64 * lh + 4 * (lr & 15);
  }
  struct WStage {
    uint4 c0[RW], c1[RW];
    uint32_t s[RW];
  };
  // every load of the main loop is unconditional (chunks past the last are
  // clamped to it: loaded, never used), so the compiler counts the loads in
  // flight and waits only for the ones a step uses
  auto load_w = [&](int q, WStage& S) {
    const int64_t c = min(q, KC - 1);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      // plain (cached) loads: the other token groups of the super-tile reuse these tiles from L2
      S.c0[i] = ld16(cl[i] + c * 1024);
      S.c1[i] = ld16(cl[i] + c * 1024 + 256);
      S.s[i] = *reinterpret_cast<const uint32_t*>(sl[i] + c * 128);
    }
  };
  // Activation fragment f = 8 g + 2 j + q of a chunk: lane l holds token
  // m0 + 32 g + (l % 32), k = 32 j + 16 (l / 32) + 8 q .. + 7 of the chunk.
  // Offsets are bytes from this token group's first row, through a buffer
  // descriptor (32-bit offsets: the host keeps 256 K below 2^31); a piece past
  // K gets an offset with bit 31 set and reads as zero (K % 16 == 0: a piece
  // is all in or out); tokens past M are clamped to the last one (never stored).
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + (int64_t)m0 * K), 0, (int)(2u * (uint32_t)min(kPfTok, M - m0) * (uint32_t)K),
      kBufferWord3);
  uint32_t xoff[FPW];
#pragma unroll
  for (int u = 0; u < FPW; ++u) {
    const int f = wave * FPW + u, g = f >> 3, jf = (f >> 1) & 3, q = f & 1;
    const int tok = min(m0 + 32 * g + lr, M - 1) - m0;
    xoff[u] = 2u * ((uint32_t)tok * (uint32_t)K + (uint32_t)(32 * jf + 16 * lh + 8 * q));
  }
  auto load_x = [&](int c, int slab) {
    c = min(c, KC - 1);
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int f = wave * FPW + u, jf = (f >> 1) & 3, q = f & 1;
      const uint32_t past = 128 * c + 32 * jf + 16 * lh + 8 * q < K ? 0u : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr)(xs[slab] + f * 1024), 16,
                                               (int)((xoff[u] + 256u * (uint32_t)c) | past), 0, 0, 0);
    }
  };

  f32x16 acc[RW][TG];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][g][v] = 0.0f;

  // step st = 2 j + q of a chunk: weight word j of c_q, activation fragments (g, j, q)
  auto read_b = [&](int slab, int st, bf16x8 (&bv)[TG]) {
    const uint8_t* xb = xs[slab] + 16 * lane;
#pragma unroll
    for (int g = 0; g < TG; ++g) bv[g] = *reinterpret_cast<const bf16x8*>(xb + (8 * g + st) * 1024);
  };
  auto deq_a = [&](const WStage& S, const float (&sc)[RW][4], int st, bf16x8 (&av)[RW]) {
    const int jj = st >> 1, q = st & 1;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const uint4& cw = q == 0 ? S.c0[i] : S.c1[i];
      const uint32_t word = jj == 0 ? cw.x : jj == 1 ? cw.y : jj == 2 ? cw.z : cw.w;
      av[i] = dequant8(word, sc[i][jj]);
    }
  };
  auto compute = [&](int slab, const WStage& S) {
    float sc[RW][4];
#pragma unroll
    for (int i = 0; i < RW; ++i) scale4(S.s[i], sc[i]);
    bf16x8 av[2][RW], bv[2][TG];
    read_b(slab, 0, bv[0]);
    deq_a(S, sc, 0, av[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int cur = st & 1;
      if (st < 7) {
        read_b(slab, st + 1, bv[cur ^ 1]);
        deq_a(S, sc, st + 1, av[cur ^ 1]);
      }
#pragma unroll
      for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int g = 0; g < TG; ++g) acc[i][g] = mfma32x32x16(av[cur][i], bv[cur][g], acc[i][g]);
    }
  };

  // chunk q is read from slab q % 2; after the barrier of iteration q (this
  // wave's loads of chunk q have landed, and every wave is done with chunk
  // q - 1) chunk q + 1 is loaded into the other slab and the weights of
  // chunk q + D - 1 into the stage chunk q - 1 used
  static_assert(D >= 2 && D <= 3, "two or three weight stages");
  WStage ws[D];
#pragma unroll
  for (int u = 0; u < D - 1; ++u) load_w(u, ws[u]);
  load_x(0, 0);
  for (int q0 = 0; q0 < KC; q0 += 2 * D) {
#pragma unroll
    for (int u = 0; u < 2 * D; ++u) {
      const int q = q0 + u;
      if (q >= KC) break;  // uniform across the workgroup
      __syncthreads();
      load_x(q + 1, (u + 1) & 1);
      load_w(q + D - 1, ws[(u + D - 1) % D]);
      compute(u & 1, ws[u % D]);
    }
  }

  // Epilogue: acc *= s_t, then t B^T is accumulated onto it by MFMA, 16
  // ranks per step (lane (lr, lh) takes ranks j0 + 8 lh .. + 7; t, its
  // K-slices summed in order, split into bf16 hi + lo parts)
  const float st = *tensor_scale;
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int g = 0; g < TG; ++g) acc[i][g] *= st;
  if (r > 0) {
    const int64_t tstride = (int64_t)M * r;
    for (int j0 = 0; j0 < r; j0 += 16) {
      const int jj = j0 + 8 * lh;
      uint4 bw[RW];
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int na = min(nw + 32 * i + lr, N - 1);
        bw[i] = make_uint4(0, 0, 0, 0);
        if (jj < r) {
          if ((r & 7) == 0) {
            bw[i] = ld16(lb + (int64_t)na * r + jj);
          } else {
            uint32_t hv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = jj + e < r ? lb[(int64_t)na * r + jj + e] : 0u;
            bw[i] = make_uint4(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16));
          }
        }
      }
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        const float* tp = t + (int64_t)min(m0 + 32 * g + lr, M - 1) * r + jj;
        float tv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int z = 0; z < tks; ++z) {
          if ((r & 3) == 0) {  // 16-byte loads: (m r + jj) is a multiple of 4
            const float* tz = tp + (int64_t)z * tstride;
            if (jj < r) {
              const f32x4 v = *reinterpret_cast<const f32x4*>(tz);
              tv[0] += v[0]; tv[1] += v[1]; tv[2] += v[2]; tv[3] += v[3];
            }
            if (jj + 4 < r) {
              const f32x4 v = *reinterpret_cast<const f32x4*>(tz + 4);
              tv[4] += v[0]; tv[5] += v[1]; tv[6] += v[2]; tv[7] += v[3];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (jj + e < r) tv[e] += tp[(int64_t)z * tstride + e];
          }
        }
        uint4 th, tl;
        split_bf16x8(tv, th, tl);
#pragma unroll
        for (int i = 0; i < RW; ++i) {
          acc[i][g] = mfma32x32x16(as_bf16x8(bw[i]), as_bf16x8(th), acc[i][g]);
          acc[i][g] = mfma32x32x16(as_bf16x8(bw[i]), as_bf16x8(tl), acc[i][g]);
        }
      }
    }
  }
  // lane holds token m0 + 32 g + lr, features nw + 32 i + 8 b + 4 lh + e (register 4 b + e)
  const bool nvec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int g = 0; g < TG; ++g) {
      const int m = m0 + 32 * g + lr;
      if (m >= M) continue;
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) {
        const int nf = nw + 32 * i + 8 * bq + 4 * lh;
        uint16_t* yp = y + (int64_t)m * N + nf;
        const f32x16& v = acc[i][g];
        const uint32_t o01 = pack_bf16x2(v[4 * bq], v[4 * bq + 1]), o23 = pack_bf16x2(v[4 * bq + 2], v[4 * bq + 3]);
        if (nvec && nf + 3 < N) {
          *reinterpret_cast<uint2*>(yp) = make_uint2(o01, o23);
        } else {
          const uint32_t o[4] = {o01 & 0xFFFFu, o01 >> 16, o23 & 0xFFFFu, o23 >> 16};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nf + e < N) yp[e] = (uint16_t)o[e];
        }
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
//   loop so their load latency overlaps it; when t is made by producer
//   workgroups of the same launch, it is staged after the main loop, once
//   their ready flag is seen.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int MTOK, int WAVES, int U>
__global__ __launch_bounds__(WAVES * kWave) void gemv_kernel(
    const uint16_t* __restrict__ x, int M, int N, int K, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ tensor_scale, const float* __restrict__ t,
    int tks, const uint16_t* __restrict__ lb, int r, uint16_t* __restrict__ y, LoraFuse lf) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t pflag;
  if ((int)blockIdx.x < lf.producers) {  // fused LoRA down-projection (the launch gives >= WAVES KB of LDS)
    lora_produce<WAVES>(lf, blockIdx.x, x, M, K, r, reinterpret_cast<f32x4*>(smem), &pflag);
    return;
  }
  const bool fused = lf.producers > 0;  // t comes from this launch: staged after the main loop
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const int KC = (K + 127) >> 7, Kp = KC * 128;
  const int rt = blockIdx.x - lf.producers;
  const int nchunk = KC;
  const int mine = nchunk > wave ? (nchunk - wave + WAVES - 1) / WAVES : 0;
  const uint8_t* cbase = codes + (int64_t)rt * KC * 1024;
  const uint8_t* sbase = scales + (int64_t)rt * KC * 128;
  const uint32_t clane = 16 * lane, slane = 4 * (16 * (lg >> 1) + li);

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
      G.sw[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sbase + (int64_t)c * 128 + slane));
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
  if (!fused) {
    for (int i = threadIdx.x; i < MTOK * r; i += WAVES * kWave) {
      const int m = i / r, j = i - m * r;
      float a = 0.0f;
      if (m < M)
        for (int q = 0; q < tks; ++q) a += t[q * tstride + (int64_t)m * r + j];  // slice order
      tsum[i] = a;
    }
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
          xv[m][q] = *reinterpret_cast<const uint4*>(xs + m * Kp + 128 * c + 32 * q + 8 * lg);
      float sc[4];
      scale4(G.sw[u], sc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // word q: 8 codes, half of one block
        const uint32_t w = G.cw[u][q];
        const bf16x2 g0v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
        const bf16x2 g1v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
        const bf16x2 g2v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
        const bf16x2 g3v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
#pragma unroll
        for (int m = 0; m < MTOK; ++m) {
          const uint4 xq = xv[m][q];  // x[k .. k+7] of this word's 8 codes
          float p = __builtin_amdgcn_fdot2_f32_bf16(g0v, __builtin_bit_cast(bf16x2, xq.x), 0.0f, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(g1v, __builtin_bit_cast(bf16x2, xq.y), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(g2v, __builtin_bit_cast(bf16x2, xq.z), p, false);
          p = __builtin_amdgcn_fdot2_f32_bf16(g3v, __builtin_bit_cast(bf16x2, xq.w), p, false);
          acc[m] = fmaf(sc[q], p, acc[m]);
        }
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
  const uint32_t t_seen = lora_poll(lf, rt);
  if (lg == 0) {
#pragma unroll
    for (int m = 0; m < MTOK; ++m) red[(wave * MTOK + m) * 16 + li] = acc[m];
  }
  __syncthreads();
  uint32_t released = 0u;
  if (fused) {  // wait for t, then stage it (one slice, coherent loads)
    lora_wait(lf, rt, t_seen);
    released = lora_release(lf, rt);
    const __amdgpu_buffer_rsrc_t trs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(t), 0, 4 * M * r, kBufferWord3);
    for (int i = threadIdx.x; i < MTOK * r; i += WAVES * kWave) tsum[i] = i < M * r ? ld_coherent4(trs, 4 * i) : 0.0f;
    __syncthreads();
  }
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
  if (fused) lora_reset_if_last(lf, rt, released);
}

size_t gemv_lds_bytes(int mtok, int64_t k, int64_t r, int waves) {
  const int64_t kp = (k + 127) / 128 * 128;
  return (size_t)(mtok * kp * 2 + (mtok * r + 16 * r) * 4 + waves * mtok * 16 * 4);
}


// More than 128 tokens: the prefill GEMM (128-token tiles, each weight
// dequantised once per 128 tokens).
static bool use_prefill(int64_t m) {
  return m > 128;
}

struct SkinnyCfg {
  int mt, nt, waves;
};

// Token tiles (16*mt) cover M; row tiles per workgroup (nt) grow with M so the
// activation fragments a lane loads are reused across more weight rows; the
// waves per workgroup split K so that ~4k waves are in flight (16 per CU),
// within a 64 KB LDS reduction buffer (waves * nt * mt <= 64).
// 3..16 tokens (one 16-token tile).
SkinnyCfg pick_skinny(int64_t m, int64_t n, int64_t k) {
  (void)m;
  const int64_t kc = (k + 127) / 128;
  if (n >= 4096) {
    // wide matrices: two row tiles share each activation fragment (halves the
    // activation re-reads); 4 waves when that still leaves >= 512 workgroups
    const int64_t groups = (n + 31) / 32;
    const int w = (int)std::min<int64_t>(groups >= 512 ? 4 : 8, std::max<int64_t>(1, kc));
    int wp = 1;
    while (wp * 2 <= w) wp *= 2;
    return SkinnyCfg{1, 2, wp};
  }
  const int64_t groups = (n + 15) / 16;
  const int wmax = (int)std::min<int64_t>(16, std::max<int64_t>(1, kc));
  int w = 1;
  // (doubling also keeps at least four chunks per wave: o 3584 -> 3584 at 8
  // tokens 7.5 -> 7.0 us with 4 waves instead of 16)
  while (w * 2 <= wmax && groups * w < 4096 && 8 * w <= kc) w *= 2;
  return SkinnyCfg{1, 1, w};
}

template <int MT, int NT, int W>
hipError_t run_skinny(dim3 grid, hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes,
                      const uint8_t* scales, const float* ts, const float* t, int tks, const uint16_t* b, int r,
                      uint16_t* y, LoraFuse lf) {
  if (lf.producers > 0 && grid.y != 1) return hipErrorInvalidValue;  // producers index grid.x
  lf.consumers = (int)(grid.x * grid.y);
  lf.groups = std::min(kLoraGroups, lf.consumers);
  hipLaunchKernelGGL((skinny_kernel<MT, NT, W>), dim3(grid.x + lf.producers, grid.y), dim3(W * kWave), 0, st, x, M, N,
                     K, codes, scales, ts, t, tks, b, r, y, lf);
  return hipGetLastError();
}

template <int MT, int NT>
hipError_t run_skinny_w(int w, dim3 grid, hipStream_t st, const uint16_t* x, int M, int N, int K,
                        const uint8_t* codes, const uint8_t* scales, const float* ts, const float* t, int tks,
                        const uint16_t* b, int r, uint16_t* y, const LoraFuse& lf) {
  // only waves * MT * NT <= 64 is instantiated: the reduction buffer is at most 64 KB of LDS
#define FP4RL_CASE(W_)                                                                             \
  case W_:                                                                                         \
    if constexpr (W_ * MT * NT <= 64 && (W_ < 16 || MT == 1)) return run_skinny<MT, NT, W_>(grid, st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, lf); \
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
  if (use_prefill(m)) return 1;  // prefill: token tiles already fill the chip
  // Up to 8 K-slices of at least 512 k (the linear's epilogue adds them in
  // order): enough workgroups for a long K without a separate reduction.
  const int64_t by_k = std::max<int64_t>(1, k / 512);
  return (int)std::min<int64_t>(8, by_k);
}

static int64_t slice_len(int64_t k, int splits) { return lora_slice_len(k, splits); }

hipError_t launch_lora_down(const uint16_t* x, int64_t m, int64_t k, const uint16_t* a, int64_t r, float lora_scale,
                            int splits, float* part, hipStream_t stream) {
  const int64_t ks = slice_len(k, splits);
  const dim3 grid((unsigned)((m + 15) / 16), (unsigned)((r + 15) / 16), (unsigned)((k + ks - 1) / ks));
  if (use_prefill(m) && r <= 128) {
    // many token tiles: a workgroup takes 32 tokens and computes every rank
    // tile, so each activation row is read once and each adapter fragment
    // feeds two token tiles (the adapter rows are re-read from L2 once per
    // 32 tokens); 8 waves with several steps of loads each in flight
    const dim3 g2((unsigned)((m + 31) / 32), 1, grid.z);
    const int rtn = (int)((r + 15) / 16);
#define FP4RL_ROWS(RTN_, U_)                                                                                     \
  if (rtn <= RTN_) {                                                                                              \
    hipLaunchKernelGGL((lora_down_rows_kernel<8, 2, RTN_, U_>), g2, dim3(8 * kWave), 0, stream, x, (int)m, (int)k, a, \
                       (int)r, lora_scale, (int)ks, part);                                                        \
    return hipGetLastError();                                                                                     \
  }
    FP4RL_ROWS(1, 8) FP4RL_ROWS(2, 4) FP4RL_ROWS(4, 2)
#undef FP4RL_ROWS
    if (rtn <= 8) {  // four waves: the reduction buffer stays at 64 KB
      hipLaunchKernelGGL((lora_down_rows_kernel<4, 2, 8, 1>), g2, dim3(4 * kWave), 0, stream, x, (int)m, (int)k, a,
                         (int)r, lora_scale, (int)ks, part);
      return hipGetLastError();
    }
  }
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
// Waves per row tile: as many as keep the whole grid resident in one round
// (up to about 8192 waves, eight per SIMD) while every wave keeps at least
// four chunks, so every wave issues all its loads at once and the kernel
// pays its load -> reduce -> store latency chain once (measured: gate
// 3584 -> 18944 14.2 -> 12.8 us with 4 waves per tile instead of 2; o
// 3584 -> 3584 7.3 -> 7.1 us with 4 instead of 16).
static int gemv_waves(int64_t n, int64_t k) {
  const int64_t rt = (n + 15) / 16, kc = (k + 127) / 128;
  int w = 1;
  while (w < 16 && 8 * w <= kc && rt * w * 2 <= 8192) w *= 2;  // doubling keeps >= 4 chunks per wave
  return w;
}

static bool use_gemv(int64_t m, int64_t n, int64_t k, int64_t r) {
  return m <= 2 && gemv_lds_bytes((int)m, k, r, gemv_waves(n, k)) <= 65536;
}

template <int MTOK, int W>
hipError_t run_gemv(hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes, const uint8_t* scales,
                    const float* ts, const float* t, int tks, const uint16_t* b, int r, uint16_t* y, LoraFuse lf) {
  constexpr int U = 4;
  size_t lds = gemv_lds_bytes(MTOK, K, r, W);
  if (lf.producers > 0) lds = std::max(lds, (size_t)W * kWave * sizeof(float) * 4);  // producers' reduction
  lf.consumers = (N + 15) / 16;
  lf.groups = std::min(kLoraGroups, lf.consumers);
  hipLaunchKernelGGL((gemv_kernel<MTOK, W, U>), dim3((unsigned)(lf.consumers + lf.producers)), dim3(W * kWave), lds, st,
                     x, M, N, K, codes, scales, ts, t, tks, b, r, y, lf);
  return hipGetLastError();
}

template <int MTOK>
hipError_t run_gemv_w(int w, hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes,
                      const uint8_t* scales, const float* ts, const float* t, int tks, const uint16_t* b, int r,
                      uint16_t* y, const LoraFuse& lf) {
  switch (w) {
    case 1: return run_gemv<MTOK, 1>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, lf);
    case 2: return run_gemv<MTOK, 2>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, lf);
    case 4: return run_gemv<MTOK, 4>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, lf);
    case 8: return run_gemv<MTOK, 8>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, lf);
    case 16: return run_gemv<MTOK, 16>(st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, lf);
    default: return hipErrorInvalidValue;
  }
}

// Split-K MFMA path: 16 < m <= 128 (decode-shaped batches).
// TM = 4 row tiles (64 features; 2 for narrow matrices with short K) per
// workgroup, TN token tiles (32 tokens per workgroup, more go to further
// token groups), W = 4 waves. K is split over
// grid.z until about 256 workgroups are in flight, while every wave keeps at
// least one chunk and the fp32 partials (written and read once) stay within
// a third of the weight bytes.
struct SplitkCfg {
  int tn, w, s, cpz, gx, gy, d, tm;
};

static bool use_splitk(int64_t m) { return m > 16 && !use_prefill(m); }

// Mid-batch kernel: eight waves per workgroup, 4 x 2 waves of 32 features
// x 64 tokens (128 features x 128 tokens per workgroup; 97..127 tokens use
// the same tile, the rows past M clamped and never stored), one workgroup
// per 128 features over all of K. Used where it beats the split-K kernel,
// which fetches and dequantises each weight tile once per 32 tokens: more
// than 96 tokens and at least 200 row groups, so that no K split is needed
// (measured, 27648 x 5120 at 112 and 128 tokens: 63 vs 73 us; at 65..96
// tokens the two are level, and narrower matrices, which would need a K
// split, are faster on the split-K kernel).
// Prefill workgroup shape: eight waves (512 features, one workgroup per CU)
// move a third fewer bytes per flop through each CU than two four-wave
// workgroups, but come in half as many, coarser pieces. A launch runs in
// rounds of 256 workgroups (one per CU); eight waves are used when rounding
// the workgroup count up to whole rounds wastes at most 1/7 of a round's
// work, else four, whose pairs per CU also run a thin last round faster.
// (Measured at 8192 tokens: 7B gate 1021 -> 1007 us, down 1113 -> 985, o 226
// -> 208, 14B gate 1040 -> 980, 32B gate 2011 -> 1942; kept on four waves:
// 7B qkv, 576 workgroups, 273 against 304 us, and 32B o, 640, 391 against
// 421; at 4096 tokens 7B down 545 -> 510, and up to 2048 tokens four waves
// throughout.)
static int prefill_waves(int64_t m, int64_t n) {
  const int64_t tiles = (n + 511) / 512 * ((m + kPfTok - 1) / kPfTok);
  const int64_t rounds = (tiles + 255) / 256;
  return 7 * 256 * rounds <= 8 * tiles ? 8 : 4;
}

constexpr int kMidRows = 128;
static bool use_mid(int64_t m, int64_t n) {
  return m > 96 && m <= 128 && (n + kMidRows - 1) / kMidRows >= 200;
}

static hipError_t launch_mid(hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes,
                             const uint8_t* scales, const float* ts, const float* t, int tks, const uint16_t* b, int r,
                             uint16_t* y, LoraFuse lf) {
  const int gx = (N + kMidRows - 1) / kMidRows;
  if (lf.producers > 0 && lf.slices > 1) {
    // one K slice per tile of t: each producer holds the kernel's LDS like a
    // main workgroup, so a few long producers run beside the row groups
    // instead of many short ones filling the chip before them (measured:
    // 32B gate at 128 tokens, r = 64: 32 producers instead of 256)
    lf.slices = 1;
    lf.kslice = K;
    lf.producers = (lf.mtiles * lf.rtiles + 7) / 8 * 8;
  }
  lf.consumers = gx;  // one waiting workgroup per row group
  lf.groups = std::min(kLoraGroups, lf.consumers);
  const unsigned grid = (unsigned)(lf.producers + gx);
  hipLaunchKernelGGL((mid_kernel<1, 2, 4, 2, 3>), dim3(grid), dim3(8 * kWave), 0, st, x, M, N, K, codes, scales, ts, t,
                     tks, b, r, y, lf);
  return hipGetLastError();
}

// Mid-batch kernel with a K split (96 < m <= 128, fewer than 200 row groups
// of 128 and long K, e.g. 32B down): every weight tile is still dequantised
// once for all the tokens; each row group's K is split into s ranges so that
// about 240 workgroups run, each writes s_t times its sums as fp32 partials,
// and a finishing launch adds the ranges and the LoRA term (t from a separate
// down-projection). The in-kernel alternative, the last workgroup of a tile
// adding the ranges, left that sum to one CU per tile.
struct MidSplit {
  int s, cps;
};
// (measured at 128 tokens: 32B down, 27648 k, 91 -> 80 us; 7B down, 18944 k,
// 50 -> 52 us, so K of at least 192 chunks)
static bool use_mid_split(int64_t m, int64_t n, int64_t k) {
  return m > 96 && m <= 128 && (n + kMidRows - 1) / kMidRows < 200 && (k + 127) / 128 >= 192;
}
static MidSplit pick_mid_split(int64_t n, int64_t k) {
  const int64_t gx = (n + kMidRows - 1) / kMidRows, kc = (k + 127) / 128;
  const int64_t s = std::max<int64_t>(1, std::min<int64_t>((240 + gx - 1) / gx, kc / 16));
  MidSplit c;
  c.cps = (int)((kc + s - 1) / s);
  c.s = (int)((kc + c.cps - 1) / c.cps);  // no empty K range
  return c;
}

static SplitkCfg pick_splitk(int64_t m, int64_t n, int64_t k) {
  SplitkCfg c;
  c.tn = 2;
  c.w = 4;
  c.gy = (int)((m + 16 * c.tn - 1) / (16 * c.tn));
  const int64_t kc = (k + 127) / 128;
  // Narrow, short matrices (at most one 64-feature tile per CU, K <= 8192):
  // two row tiles per wave, so twice the workgroups share the work without
  // splitting K further (measured: o 3584 -> 3584 at 32 tokens 13.7 -> 10.0
  // us). Long K keeps four row tiles: its K splits already fill the chip.
  c.tm = (n + 63) / 64 * c.gy <= 256 && kc <= 64 ? 2 : 4;
  c.gx = (int)((n + 16 * c.tm - 1) / (16 * c.tm));
  const double wbytes = (double)n * (double)k * 0.5625;
  int s = 1;
  while ((int64_t)c.gx * c.gy * s < 256 && (kc + 2 * s - 1) / (2 * s) >= c.w &&
         4.0 * (double)(2 * s) * (double)m * (double)n * 2.0 <= wbytes / 3.0)
    s *= 2;
  // Long K: split further until each wave has at most 24 chunks, within the
  // same bound on the partials (measured: 32B down, 27648 k, at 128 tokens
  // 108 -> 89 us with three ranges; 320 output tiles had left it unsplit)
  while (s < 8 && (kc + (int64_t)s * c.w - 1) / ((int64_t)s * c.w) > 24 &&
         4.0 * (double)(s + 1) * (double)m * (double)n * 2.0 <= wbytes / 3.0)
    ++s;
  c.cpz = (int)((kc + s - 1) / s);
  c.s = (int)((kc + c.cpz - 1) / c.cpz);  // no empty K range
  if ((int64_t)c.gx * c.gy > kSplitCounters) c.s = 1, c.cpz = (int)kc;  // a split needs one counter per tile
  // more output tiles than CUs (wide matrices) or long K: the lighter
  // pipeline at three waves per SIMD; otherwise the deeper one, which hides
  // latency at one wave per SIMD (measured: gate 3584 -> 18944 at 64 tokens
  // 28.8 -> 26.1 us, down 18944 -> 3584 at 32 tokens 22.9 -> 21.8 us, while
  // o 3584 -> 3584 is 1 us slower with it)
  c.d = (int64_t)c.gx * c.gy > 256 || kc > 64 ? 2 : 3;
  return c;
}

size_t linear_partial_bytes(int64_t m, int64_t n, int64_t k) {
  if (use_mid_split(m, n, k))
    return ((size_t)pick_mid_split(n, k).s * (size_t)m * (size_t)n * sizeof(float) + 255) / 256 * 256;
  if (use_mid(m, n) || !use_splitk(m)) return 0;
  const SplitkCfg c = pick_splitk(m, n, k);
  if (c.s == 1) return 0;
  return ((size_t)c.s * (size_t)m * (size_t)n * sizeof(float) + 255) / 256 * 256;
}

template <int TN, int W, int D, int TM = 4>
hipError_t run_splitk(const SplitkCfg& c, hipStream_t st, const uint16_t* x, int M, int N, int K, const uint8_t* codes,
                      const uint8_t* scales, const float* ts, const float* t, int tks, const uint16_t* b, int r,
                      uint16_t* y, float* part, uint32_t* counters, LoraFuse lf) {
  // the partials are addressed with 32-bit byte offsets (at most 1024 tiles of
  // 64 x 32 outputs are split, so they stay far below this bound)
  if (c.s > 1 && (int64_t)c.s * M * N * 4 > INT32_MAX) return hipErrorInvalidValue;
  const int main_grid = 8 * ((c.gx + 7) / 8) * c.gy * c.s;
  lf.consumers = c.gx * c.gy;  // one waiting workgroup per output tile (the last of its K split)
  lf.groups = std::min(kLoraGroups, lf.consumers);
  const unsigned grid = (unsigned)(lf.producers + main_grid);
  hipLaunchKernelGGL((splitk_kernel<TM, TN, W, D>), dim3(grid), dim3(W * kWave), 0, st, x, M, N, K, codes, scales, ts, t,
                     tks, b, r, y, c.cpz, c.s, c.s > 1 ? part : nullptr, c.s > 1 ? counters : nullptr, lf);
  return hipGetLastError();
}

static hipError_t launch_splitk(const SplitkCfg& c, hipStream_t st, const uint16_t* x, int M, int N, int K,
                                const uint8_t* codes, const uint8_t* scales, const float* ts, const float* t, int tks,
                                const uint16_t* b, int r, uint16_t* y, float* part, uint32_t* counters,
                                const LoraFuse& lf) {
#define FP4RL_SPLITK(TN_, W_)                                                                              \
  if (c.tn == TN_ && c.w == W_ && c.d == 2)                                                                 \
    return run_splitk<TN_, W_, 2>(c, st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, part, counters, lf); \
  if (c.tn == TN_ && c.w == W_ && c.d == 3)                                                                 \
    return run_splitk<TN_, W_, 3>(c, st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, part, counters, lf);
  if (c.tm == 2 && c.tn == 2 && c.w == 4 && c.d == 2)
    return run_splitk<2, 4, 2, 2>(c, st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, part, counters, lf);
  if (c.tm == 2 && c.tn == 2 && c.w == 4 && c.d == 3)
    return run_splitk<2, 4, 3, 2>(c, st, x, M, N, K, codes, scales, ts, t, tks, b, r, y, part, counters, lf);
  if (c.tm != 4) return hipErrorInvalidValue;
  FP4RL_SPLITK(2, 4)
#undef FP4RL_SPLITK
  return hipErrorInvalidValue;
}

// FP8 (E4M3) decode, 17..64 tokens: the split-K kernel's F8 mode (y, or
// with a K split fp32 partials [s][m][n] times the row scales, which the FP8
// linear's finishing launch adds with the LoRA term). Two 16-token tiles per
// workgroup, K split as for NVFP4 weights (their bytes are n k here).
static SplitkCfg pick_fp8_splitk(int64_t m, int64_t n, int64_t k) {
  SplitkCfg c;
  c.tn = 2;
  c.w = 4;
  c.gy = (int)((m + 16 * c.tn - 1) / (16 * c.tn));
  const int64_t kc = (k + 127) / 128;
  c.tm = (n + 63) / 64 * c.gy <= 256 && kc <= 64 ? 2 : 4;
  c.gx = (int)((n + 16 * c.tm - 1) / (16 * c.tm));
  const double wbytes = (double)n * (double)k;
  int s = 1;
  while ((int64_t)c.gx * c.gy * s < 256 && (kc + 2 * s - 1) / (2 * s) >= c.w &&
         4.0 * (double)(2 * s) * (double)m * (double)n * 2.0 <= wbytes / 3.0)
    s *= 2;
  while (s < 8 && (kc + (int64_t)s * c.w - 1) / ((int64_t)s * c.w) > 24 &&
         4.0 * (double)(s + 1) * (double)m * (double)n * 2.0 <= wbytes / 3.0)
    ++s;
  c.cpz = (int)((kc + s - 1) / s);
  c.s = (int)((kc + c.cpz - 1) / c.cpz);
  c.d = (int64_t)c.gx * c.gy > 256 || kc > 64 ? 2 : 3;
  return c;
}

int fp8_splitk_slices(int64_t m, int64_t n, int64_t k) { return pick_fp8_splitk(m, n, k).s; }

hipError_t launch_fp8_splitk(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                             const float* scales, const float* t, int tks, const uint16_t* b, int64_t r, uint16_t* y,
                             float* part, const float* tok_scale, hipStream_t stream) {
  const SplitkCfg c = pick_fp8_splitk(m, n, k);
  const unsigned grid = (unsigned)(8 * ((c.gx + 7) / 8) * c.gy * c.s);
  const uint8_t* sc = reinterpret_cast<const uint8_t*>(scales);
#define FP4RL_F8(TM_, TN_, D_)                                                                                       \
  if (c.tm == TM_ && c.tn == TN_ && c.d == D_) {                                                                      \
    hipLaunchKernelGGL((splitk_kernel<TM_, TN_, 4, D_, true>), dim3(grid), dim3(4 * kWave), 0, stream, x, (int)m,     \
                       (int)n, (int)k, codes, sc, scales, t, tks, b, (int)r, y, c.cpz, c.s, part, nullptr,            \
                       LoraFuse{}, tok_scale);                                                                        \
    return hipGetLastError();                                                                                         \
  }
  FP4RL_F8(4, 2, 2) FP4RL_F8(4, 2, 3) FP4RL_F8(2, 2, 2) FP4RL_F8(2, 2, 3)
#undef FP4RL_F8
  return hipErrorInvalidValue;
}

const char* fp4_linear_kernel_name(int64_t m, int64_t n, int64_t k, int64_t r) {
  static const char* const kNames[2][5] = {
#define FP4RL_NAME_ROW(MT_, NT_)                                                                           \
  {"skinny_kernel<" #MT_ ", " #NT_ ", 1>", "skinny_kernel<" #MT_ ", " #NT_ ", 2>",                          \
   "skinny_kernel<" #MT_ ", " #NT_ ", 4>", "skinny_kernel<" #MT_ ", " #NT_ ", 8>",                          \
   "skinny_kernel<" #MT_ ", " #NT_ ", 16>"}
      FP4RL_NAME_ROW(1, 1), FP4RL_NAME_ROW(1, 2),
#undef FP4RL_NAME_ROW
  };
  static const char* const kGemv[2][5] = {
      {"gemv_kernel<1, 1, 4>", "gemv_kernel<1, 2, 4>", "gemv_kernel<1, 4, 4>", "gemv_kernel<1, 8, 4>",
       "gemv_kernel<1, 16, 4>"},
      {"gemv_kernel<2, 1, 4>", "gemv_kernel<2, 2, 4>", "gemv_kernel<2, 4, 4>", "gemv_kernel<2, 8, 4>",
       "gemv_kernel<2, 16, 4>"}};
  if (use_gemv(m, n, k, r)) {
    int wi = 0;
    while ((1 << wi) < gemv_waves(n, k)) ++wi;
    return kGemv[m - 1][wi];
  }
  if (use_prefill(m)) return prefill_waves(m, n) == 8 ? "prefill_kernel<2, 8>" : "prefill_kernel<2, 4>";
  if (use_mid(m, n) || use_mid_split(m, n, k)) return "mid_kernel<1, 2, 4, 2, 3>";
  if (use_splitk(m)) {
    const SplitkCfg sc = pick_splitk(m, n, k);
    static const char* const kSplitk[3][2] = {{"splitk_kernel<2, 2, 4, 2>", "splitk_kernel<2, 2, 4, 3>"},
                                              {"splitk_kernel<4, 2, 4, 2>", "splitk_kernel<4, 2, 4, 3>"},
                                              {"splitk_kernel<4, 4, 4, 2>", "splitk_kernel<4, 4, 4, 3>"}};
    return kSplitk[sc.tm == 2 ? 0 : sc.tn == 2 ? 1 : 2][sc.d == 2 ? 0 : 1];
  }
  const SkinnyCfg c = pick_skinny(m, n, k);
  int wi = 0;
  while ((1 << wi) < c.waves) ++wi;
  return kNames[c.nt == 1 ? 0 : 1][wi];
}

bool linear_fuses_lora(int64_t m, int64_t n, int64_t k) {
  // every decode kernel (GEMV, skinny: one token group; split-K; mid-batch)
  // but the mid-batch kernel's K split, whose finishing launch adds t B^T
  return !use_prefill(m) && !use_mid_split(m, n, k);
}

int64_t lora_slice_len(int64_t k, int splits) { return ((k + splits - 1) / splits + 31) / 32 * 32; }

hipError_t launch_fp4_linear(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* codes,
                             const uint8_t* scales, const float* tensor_scale, const float* t, int tks,
                             const uint16_t* b, int64_t r, uint16_t* y, float* part, uint32_t* counters,
                             LoraFuse lf, hipStream_t stream) {
  if (lf.producers > 0 &&
      (!linear_fuses_lora(m, n, k) || lf.mtiles * lf.rtiles > kLoraTileCounters || tks != 1 || lf.slices > 8))
    return hipErrorInvalidValue;
  const int M = (int)m, N = (int)n, K = (int)k, R = (int)r;
  // the skinny kernel addresses activations with 32-bit byte offsets
  if (m > 2 && m <= 16 && 2 * m * k > INT32_MAX) return hipErrorInvalidValue;
  if (use_gemv(m, n, k, r)) {
    const int w = gemv_waves(n, k);
    return m == 1 ? run_gemv_w<1>(w, stream, x, M, N, K, codes, scales, tensor_scale, t, tks, b, R, y, lf)
                  : run_gemv_w<2>(w, stream, x, M, N, K, codes, scales, tensor_scale, t, tks, b, R, y, lf);
  }
  if (use_mid_split(m, n, k)) {
    const MidSplit c = pick_mid_split(n, k);
    if (part == nullptr || lf.producers > 0) return hipErrorInvalidValue;
    const int gx = (N + kMidRows - 1) / kMidRows;
    hipLaunchKernelGGL((mid_kernel<1, 2, 4, 2, 3>), dim3((unsigned)(gx * c.s)), dim3(8 * kWave), 0, stream, x, M, N, K,
                       codes, scales, tensor_scale, t, tks, b, R, y, LoraFuse{}, c.s, c.cps, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_partials_finish(part, c.s, m, n, r > 0 ? t : nullptr, tks, r > 0 ? b : nullptr, r, y, stream);
  }
  if (use_mid(m, n)) return launch_mid(stream, x, M, N, K, codes, scales, tensor_scale, t, tks, b, R, y, lf);
  if (use_splitk(m))
    return launch_splitk(pick_splitk(m, n, k), stream, x, M, N, K, codes, scales, tensor_scale, t, tks, b, R, y, part,
                         counters, lf);
  if (use_prefill(m)) {
    const int waves = prefill_waves(m, n);
    const int64_t gr = (n + 64 * waves - 1) / (64 * waves), gt = (m + kPfTok - 1) / kPfTok;
    const int64_t supers = (gr + 7) / 8 * ((gt + 3) / 4);  // super-tiles of 8 x 4 workgroups, dealt to 8 XCDs
    const int64_t grid = 8 * 32 * ((supers + 7) / 8);
    if (waves == 8)
      hipLaunchKernelGGL((prefill_kernel<2, 8>), dim3((unsigned)grid), dim3(512), 0, stream, x, M, N, K, codes,
                         scales, tensor_scale, t, tks, b, R, y);
    else
      hipLaunchKernelGGL((prefill_kernel<2, 4>), dim3((unsigned)grid), dim3(256), 0, stream, x, M, N, K, codes,
                         scales, tensor_scale, t, tks, b, R, y);
    return hipGetLastError();
  }
  // 3..16 tokens: one token tile, so grid.y is 1
  const SkinnyCfg cfg = pick_skinny(m, n, k);
  const dim3 grid((unsigned)((n + 16 * cfg.nt - 1) / (16 * cfg.nt)), (unsigned)((m + 16 * cfg.mt - 1) / (16 * cfg.mt)));
#define FP4RL_SKINNY(MT_, NT_) \
  if (cfg.mt == MT_ && cfg.nt == NT_) \
    return run_skinny_w<MT_, NT_>(cfg.waves, grid, stream, x, M, N, K, codes, scales, tensor_scale, t, tks, b, R, y, lf);
  FP4RL_SKINNY(1, 1) FP4RL_SKINNY(1, 2)
#undef FP4RL_SKINNY
  return hipErrorInvalidValue;
}

}  // namespace fp4rl
