// Device-side helpers shared by the gfx950 kernels of libfp4rl.
//
// Number formats (NVFP4):
//   E2M1 element code: bit 3 sign, bits 0-2 index k of g_k in {0,.5,1,1.5,2,3,4,6}.
//   E4M3 block scale: OCP e4m3fn byte, bias 7, subnormals m*2^-9, max 448.
// Every product g_k * S_b of an E2M1 magnitude and a finite E4M3 value has at
// most 6 significant bits and lies in [2^-10, 2688], so it is exact in bf16:
// kernels dequantise to bf16 without rounding and apply the fp32 tensor scale
// once, in the epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4rl {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet).
// Two fp32 -> bf16 round-to-nearest-even conversions in one instruction
// (v_cvt_pk_bf16_f32); a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Value of an E4M3 byte (sign ignored: block scales are non-negative).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// Upper halves of two fp32 values packed as (lo, hi) bf16; exact when both
// values are bf16 numbers.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// One byte of two E2M1 codes (low nibble first) -> two fp32 values g_k.
// The hardware convert applies only the exponent of its fp32 scale operand,
// so it runs at scale 1 (exact) and the E4M3 block scale is multiplied after.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Eight codes of one dword (element 2j = low nibble of byte j) times the
// block scale s -> eight bf16 values, exact.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s) {
  const f32x2 p0 = e2m1_pair<0>(w), p1 = e2m1_pair<1>(w);
  const f32x2 p2 = e2m1_pair<2>(w), p3 = e2m1_pair<3>(w);
  uint4 o;
  o.x = pack_hi16(p0.x * s, p0.y * s);
  o.y = pack_hi16(p1.x * s, p1.y * s);
  o.z = pack_hi16(p2.x * s, p2.y * s);
  o.w = pack_hi16(p3.x * s, p3.y * s);
  return __builtin_bit_cast(bf16x8, o);
}

// Streaming (non-temporal) 16- and 8-byte accesses for data touched once.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// 16 x 16 x 128 product of OCP E4M3 bytes (32 per lane, the same lane/slot
// layout for both operands), unit block scales (E8M0 127 = 2^0)
__device__ __forceinline__ f32x4 mfma16x16x128_e4m3(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ i32x8 as_i32x8(uint4 lo, uint4 hi) {
  return i32x8{(int32_t)lo.x, (int32_t)lo.y, (int32_t)lo.z, (int32_t)lo.w,
               (int32_t)hi.x, (int32_t)hi.y, (int32_t)hi.z, (int32_t)hi.w};
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Eight fp32 values split into bf16 hi + lo parts (v ~= hi + lo to ~2^-17).
__device__ __forceinline__ void split_bf16x8(const float* v, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    l[j] = pack_bf16x2(v[2 * j] - __uint_as_float(h[j] << 16), v[2 * j + 1] - __uint_as_float(h[j] & 0xFFFF0000u));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

}  // namespace fp4rl
