// MFMA GEMM with both operands contiguous along the contraction (internal
// to libfp4rl): C[m][q] = alpha qscale[q] lscale[m] sum_c L1[m][c] R1[q][c]
// (+ sum_c L2[m][c] R2[q][c]). Operands are bf16; R1 may hold OCP E4M3
// bytes, converted to bf16 (exactly) on the way into LDS, or both L1 and R1
// may hold E4M3 bytes, multiplied on the FP8 matrix cores as they are.
#pragma once

#include <algorithm>
#include <type_traits>

#include "device.hpp"

namespace fp4rl {

constexpr int kNtRsrcWord3 = 0x00020000;

// ---------------------------------------------------------------------------
// C[m][q] = alpha sum_c L1[m][c] R1[q][c] (+ sum_c L2[m][c] R2[q][c]), rows
// contiguous along c (row strides and lengths multiples of 16 bytes), fp32
// accumulation. A workgroup computes a 128 (m) x 128 (q) tile with 4 waves
// of 64 x 64 (4 x 4 MFMA tiles each) over one slice of the contraction
// (blockIdx.y; one slice unless the launch splits it).
// Contraction chunks of 128 bytes per row (64 bf16 or 128 E4M3 values) are
// loaded to registers one chunk ahead and written to one of two LDS slabs
// per operand (rows padded to 144 B: conflict-free 16-byte fragment reads);
// one barrier per chunk. Rows past M or Q are clamped (loaded, never
// stored); pieces past the slice read as zero (their offsets fall outside
// the buffer descriptor's range).
// Operand modes: kNtBf16 (bf16 x bf16: two 16x16x32 MFMA steps per chunk),
// kNtR8 (R E4M3, 64 bytes per row and chunk widened to bf16 in LDS),
// kNtE4M3 (L and R E4M3: one 16x16x128 FP8 MFMA per chunk; a lane's 32
// bytes are bytes 16 g .. + 15 and 64 + 16 g .. + 15 of its row's chunk,
// the same slots on both operands, so the sum is the plain one).
// A lane's result holds q = 4 g + v of MFMA column li = m, so stores are
// 4 consecutive outputs of one row. Outputs: bf16 y [M][Q], or fp32
// part[slice][M][Q].
// ---------------------------------------------------------------------------
constexpr int kGT = 128, kGC = 64, kGPitch = kGC + 8;
constexpr int kNtBf16 = 0, kNtR8 = 1, kNtE4M3 = 2;

struct Seg {
  const void* l = nullptr;        // [M][ld] bf16, or E4M3 bytes (kNtE4M3)
  const void* r = nullptr;        // [Q][ld] bf16, or E4M3 bytes (kNtR8, kNtE4M3)
  int ld = 0;                     // row stride of both operands (elements)
  int c = 0;                      // contraction length (0: no segment)
  int slice = 0;                  // contraction per blockIdx.y (a multiple of the chunk; >= c: unsplit)
  const float* lscale = nullptr;  // optional per-row scale of L [M] (first segment only)
};

template <bool BF16OUT, int WM, int MODE = kNtBf16>
__global__ __launch_bounds__(256) void nt_gemm_kernel(Seg s1, Seg s2, int M, int Q, const float* __restrict__ alpha_dev,
                                                      float alpha, const float* __restrict__ qscale,
                                                      uint16_t* __restrict__ ybf, float* __restrict__ part) {
  constexpr int TMM = kGT * WM;  // m rows of the workgroup tile (each wave: 64 WM x 64)
  __shared__ __align__(16) uint16_t ls[2][TMM * kGPitch];
  __shared__ __align__(16) uint16_t rs[2][kGT * kGPitch];
  const int MT = (M + TMM - 1) / TMM;
  const int mt = blockIdx.x % MT, qt = blockIdx.x / MT;
  const int m0 = TMM * mt, q0 = kGT * qt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave & 1, wq = wave >> 1;
  const int prow = threadIdx.x >> 3, pcol = threadIdx.x & 7;  // piece: rows prow + 32 i, bytes 16 pcol .. + 15

  f32x4 acc[4][4 * WM];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4 * WM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto run = [&](const Seg& S, int c0, int clen, auto mode) {
    constexpr int MD = decltype(mode)::value;
    constexpr int LB = MD == kNtE4M3 ? 1 : 2;  // bytes per L element
    constexpr int RB = MD == kNtBf16 ? 2 : 1;  // bytes per R element
    constexpr int CH = MD == kNtE4M3 ? 128 : 64;  // contraction per chunk
    constexpr int LPE = 16 / LB;                  // L elements per piece
    const int NC = (clen + CH - 1) / CH;
    const int lrows = min(TMM, M - m0), rrows = min(kGT, Q - q0);
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(S.l) + LB * ((int64_t)m0 * S.ld + c0)), 0,
        LB * ((lrows - 1) * S.ld + clen), kNtRsrcWord3);
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(S.r) + RB * ((int64_t)q0 * S.ld + c0)), 0,
        RB * ((rrows - 1) * S.ld + clen), kNtRsrcWord3);
    uint32_t loff[4 * WM], roff[4];  // roff: RP (<= 4) used
#pragma unroll
    for (int i = 0; i < 4 * WM; ++i)
      loff[i] = (uint32_t)LB * ((uint32_t)min(prow + 32 * i, lrows - 1) * (uint32_t)S.ld) + 16u * pcol;
    // 16-byte R pieces: rows prow + 32 i, bytes 16 pcol (bf16 or E4M3 x E4M3);
    // widened E4M3 (kNtR8): rows (tid >> 2) + 64 i, columns 16 (tid & 3)
    constexpr bool WIDEN = MD == kNtR8;
    constexpr int RP = WIDEN ? 2 : 4;  // R pieces per thread and chunk
    const int rrow = WIDEN ? (int)(threadIdx.x >> 2) : prow, rcol = WIDEN ? 16 * (threadIdx.x & 3) : (16 / RB) * pcol;
    constexpr int RSTEP = WIDEN ? 64 : 32;
#pragma unroll
    for (int i = 0; i < RP; ++i)
      roff[i] = (uint32_t)RB * ((uint32_t)min(rrow + RSTEP * i, rrows - 1) * (uint32_t)S.ld + rcol);
    uint4 lv[4 * WM], rv[4];  // rv: RP used
    auto load = [&](int ch) {
      ch = min(ch, NC - 1);
      const uint32_t out = CH * ch + LPE * pcol < clen ? 0u : 0x80000000u;
      const uint32_t rout = CH * ch + rcol < clen ? 0u : 0x80000000u;
#pragma unroll
      for (int i = 0; i < 4 * WM; ++i)
        lv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lrs, (int)((loff[i] + (uint32_t)LB * CH * ch) | out), 0, 0));
#pragma unroll
      for (int i = 0; i < RP; ++i)
        rv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rrs, (int)((roff[i] + (uint32_t)RB * CH * ch) | rout), 0, 0));
    };
    auto store = [&](int slab) {
#pragma unroll
      for (int i = 0; i < 4 * WM; ++i)
        *reinterpret_cast<uint4*>(&ls[slab][(prow + 32 * i) * kGPitch + 8 * pcol]) = lv[i];
#pragma unroll
      for (int i = 0; i < RP; ++i) {
        if constexpr (WIDEN) {
          // 16 E4M3 values -> 16 bf16 (exact: 4 significant bits), hardware convert at unit scale
          uint32_t o[8];
          const uint32_t w4[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w4[d], false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(w4[d], true);
            o[2 * d] = pack_hi16(lo.x, lo.y);
            o[2 * d + 1] = pack_hi16(hi.x, hi.y);
          }
          uint16_t* dst = &rs[slab][(rrow + RSTEP * i) * kGPitch + rcol];
          *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<uint4*>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
        } else {
          *reinterpret_cast<uint4*>(&rs[slab][(prow + 32 * i) * kGPitch + 8 * pcol]) = rv[i];
        }
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
      if constexpr (MD == kNtE4M3) {
        i32x8 a[4], b[4 * WM];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint16_t* p = rsl + (64 * wq + 16 * i + li) * kGPitch + 8 * lg;
          a[i] = as_i32x8(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 32));
        }
#pragma unroll
        for (int j = 0; j < 4 * WM; ++j) {
          const uint16_t* p = lsl + (64 * WM * wm + 16 * j + li) * kGPitch + 8 * lg;
          b[j] = as_i32x8(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 32));
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4 * WM; ++j) acc[i][j] = mfma16x16x128_e4m3(a[i], b[j], acc[i][j]);
        __builtin_amdgcn_s_setprio(0);
      } else {
#pragma unroll
        for (int st = 0; st < kGC / 32; ++st) {
          bf16x8 a[4], b[4 * WM];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a[i] = as_bf16x8(*reinterpret_cast<const uint4*>(rsl + (64 * wq + 16 * i + li) * kGPitch + 32 * st + 8 * lg));
#pragma unroll
          for (int j = 0; j < 4 * WM; ++j)
            b[j] = as_bf16x8(*reinterpret_cast<const uint4*>(lsl + (64 * WM * wm + 16 * j + li) * kGPitch + 32 * st + 8 * lg));
          __builtin_amdgcn_s_setprio(1);  // favour this wave's MFMA burst over waves still loading
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4 * WM; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
          __builtin_amdgcn_s_setprio(0);
        }
      }
    }
  };

  const int c0 = blockIdx.y * s1.slice;
  run(s1, c0, min(s1.slice, s1.c - c0), std::integral_constant<int, MODE>{});
  const float al = alpha_dev ? *alpha_dev : alpha;
  float msc[4 * WM];  // per-row scale of L: lane holds m = m0 + 64 WM wm + 16 j + li
#pragma unroll
  for (int j = 0; j < 4 * WM; ++j) msc[j] = s1.lscale ? s1.lscale[min(m0 + 64 * WM * wm + 16 * j + li, M - 1)] : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // per-column scale (q rows of R): lane holds q = q0 + 64 wq + 16 i + 4 g + v
    f32x4 sc = f32x4{al, al, al, al};
    if (qscale) {
      const int qb = q0 + 64 * wq + 16 * i + 4 * lg;
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = al * qscale[min(qb + v, Q - 1)];
    }
#pragma unroll
    for (int j = 0; j < 4 * WM; ++j) acc[i][j] *= sc * msc[j];
  }
  if (s2.c > 0) run(s2, 0, s2.c, std::integral_constant<int, kNtBf16>{});  // only with an unsplit first segment

  float* pout = part ? part + (int64_t)blockIdx.y * M * Q : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4 * WM; ++j) {
      const int m = m0 + 64 * WM * wm + 16 * j + li, q = q0 + 64 * wq + 16 * i + 4 * lg;
      if (m >= M) continue;
      const f32x4 v = acc[i][j];
      if constexpr (BF16OUT) {
        uint16_t* yp = ybf + (int64_t)m * Q + q;
        if (q + 3 < Q && (Q & 3) == 0) {
          *reinterpret_cast<uint2*>(yp) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (q + e < Q) yp[e] = (uint16_t)f32_to_bf16(v[e]);
        }
      } else {
        float* yp = pout + (int64_t)m * Q + q;
        if (q + 3 < Q && (Q & 3) == 0) {
          *reinterpret_cast<float4*>(yp) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (q + e < Q) yp[e] = v[e];
        }
      }
    }
}

// Contraction slices for a launch of `tiles` output tiles: enough workgroups
// to fill the chip (>= 512), each slice at least 512 long (a multiple of the
// chunk: 64 for bf16 L, 128 for E4M3 L).
inline int nt_slice_len(int64_t tiles, int64_t c, int chunk = kGC) {
  int64_t s = (512 + tiles - 1) / tiles;
  s = std::max<int64_t>(1, std::min<int64_t>(s, c / 512));
  const int64_t len = ((c + s - 1) / s + chunk - 1) / chunk * chunk;
  return (int)len;
}
inline int nt_slices(int64_t tiles, int64_t c, int chunk = kGC) {
  const int64_t len = nt_slice_len(tiles, c, chunk);
  return (int)((c + len - 1) / len);
}
inline int64_t nt_tiles(int64_t m, int64_t q) { return ((m + kGT - 1) / kGT) * ((q + kGT - 1) / kGT); }

}  // namespace fp4rl
