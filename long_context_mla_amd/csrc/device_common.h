// Device helpers shared by the gfx950 kernels: vector types, MFMA operand
// types, bf16 and E4M3 conversions, and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;   // tokens per physical cache page
constexpr int kD = 576;     // latent row: 512 latent + 64 rope
constexpr int kDV = 512;    // value = first 512 elements of the row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum CacheKind { kBf16 = 0, kFp8 = 1 };
enum ScaleKind { kScaleNone = 0, kScaleTensor = 1, kScaleToken = 2 };

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

#define MLA_LDS __attribute__((address_space(3)))
#define MLA_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ uint32_t bits_of(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float float_of(uint32_t x) { return __builtin_bit_cast(float, x); }

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_float(uint16_t b) { return float_of(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t float_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Four E4M3 bytes -> four bf16 values (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}

// Eight E4M3 bytes (little-endian in two dwords) -> MFMA bf16x8 operand, element j = byte j.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(u32x2 w) {
  bf16x2 a, b, c, d;
  e4m3x4_to_bf16(w.x, a, b);
  e4m3x4_to_bf16(w.y, c, d);
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// float -> OCP E4M3FN code: round to nearest, ties to even mantissa, saturating to
// +-448, NaN -> 0x7F with the input's sign; the sign of a zero result is kept.
// Integer formulation on the fp32 bit pattern.
__device__ __forceinline__ uint32_t float_to_e4m3(float x) {
  const uint32_t u = bits_of(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;   // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448: largest finite
  if (a >= 0x3c800000u) {                      // |x| >= 2^-6: normal E4M3 range
    a += 0x7ffffu + ((a >> 20) & 1u);          // round the 23-bit mantissa to 3 bits, ties to even
    return sign | ((a >> 20) - (120u << 3));   // rebias exponent 127 -> 7
  }
  // subnormal E4M3: multiples of 2^-9; scaling by 2^9 is exact, rint ties to even
  const float m = __builtin_rintf(float_of(a) * 512.0f);
  return sign | uint32_t(m);
}

// Wave-wide reductions over 64 lanes.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Reduction across the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float group4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace mla
