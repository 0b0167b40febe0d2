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
// Two floats -> two bf16 in one dword (lo = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
// acc + lo + hi of a dword holding two bf16 values, in fp32.
__device__ __forceinline__ float dot2_bf16_ones(uint32_t pk, float acc) {
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
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

// One new latent row in E4M3, the encoding kv_append_fp8 defines: lane l takes
// the 8-element chunks l and, for l < 8, l + 64 of the 576 bf16 values;
// codes[c] holds chunk c's eight codes (element 0 in the low byte).  PER_TOKEN
// (all 64 lanes take part): scale = amax / 448 (1 for an all-zero row);
// otherwise the given tensor_scale.  Returns the scale.
template <bool PER_TOKEN>
__device__ __forceinline__ float encode_row_e4m3(const uint16_t* row, int lane, float tensor_scale,
                                                 u32x2 (&codes)[2]) {
  const u32x4* src = reinterpret_cast<const u32x4*>(row);
  const int nchunk = lane < 8 ? 2 : 1;
  float x[2][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c < nchunk) {
      const u32x4 w = src[lane + 64 * c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][2 * e] = float_of(w[e] << 16);
        x[c][2 * e + 1] = float_of(w[e] & 0xffff0000u);
        amax = fmaxf(amax, fmaxf(fabsf(x[c][2 * e]), fabsf(x[c][2 * e + 1])));
      }
    }
  }
  float scale = tensor_scale;
  if (PER_TOKEN) {
    amax = wave_max(amax);
    scale = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    uint32_t lo = 0, hi = 0;
    if (c < nchunk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= float_to_e4m3(__fdiv_rn(x[c][e], scale)) << (8 * e);
        hi |= float_to_e4m3(__fdiv_rn(x[c][4 + e], scale)) << (8 * e);
      }
    }
    codes[c] = u32x2{lo, hi};
  }
  return scale;
}

// max(a, b, c) in one instruction.  fmaxf chains get an extra canonicalising
// max per operand that is not provably a quiet value (a masked score is a
// select), which doubles the work of a running maximum.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Reduction across the four 16-lane groups (lanes l, l^16, l^32, l^48), on
// the VALU: permlane16_swap pairs rows 0/1 and 2/3, permlane32_swap pairs the
// two halves of the wave.
__device__ __forceinline__ float group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(bits_of(v), bits_of(v), false, false);
  v = fmaxf(float_of(a[0]), float_of(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(bits_of(v), bits_of(v), false, false);
  return fmaxf(float_of(b[0]), float_of(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(bits_of(v), bits_of(v), false, false);
  v = float_of(a[0]) + float_of(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(bits_of(v), bits_of(v), false, false);
  return float_of(b[0]) + float_of(b[1]);
}

// Transposing LDS reads (gfx950).  Within each 16-lane group, lane i of the
// result holds, for j = 0..7 (b8) or 0..3 (b16), the element at offset
// (i & 7) (b8) or (i & 3) (b16) of the 8-byte row addressed by lane
// 2j + (i >> 3) (b8) or 4j + (i >> 2) (b16) of the group.
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
  typedef __attribute__((ext_vector_type(2))) int i32x2;
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)p);
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  typedef __attribute__((ext_vector_type(4))) short i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Hand-placed MFMAs.  The compiler's hazard tracking does not see inside inline
// asm, so these carry their own wait states: each pair starts with s_nop 2
// (covers a VALU or v_accvgpr_write producing a source just before), and a
// result is read by VALU or stored only after mfma_result_fence(), which
// waits out the MFMA write latency and ties the register so that no reader
// is scheduled ahead of it.  Back-to-back accumulation into the same
// registers (SrcC = vDst) needs no wait states.
//
// S^T[tok][row] += K[tok][:] . Q[row][:] for two row blocks: K in VGPRs, the
// two query operands in AGPRs, the accumulators in VGPRs.
__device__ __forceinline__ void mfma_qk2(f32x4& s0, f32x4& s1, bf16x8 k, bf16x8 q0, bf16x8 q1) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %4, %1"
      : "+v"(s0), "+v"(s1)
      : "v"(k), "a"(q0), "a"(q1));
}
// O[row][dim] += P[row][:] . V[:][dim] for two row blocks: P and V in VGPRs,
// the accumulators in AGPRs.
__device__ __forceinline__ void mfma_pv2(f32x4& o0, f32x4& o1, bf16x8 p0, bf16x8 p1, bf16x8 v) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %4, %1"
      : "+a"(o0), "+a"(o1)
      : "v"(p0), "v"(p1), "v"(v));
}
// The same for the first k-block: accumulators start from the inline constant 0.
__device__ __forceinline__ void mfma_qk2_first(f32x4& s0, f32x4& s1, bf16x8 k, bf16x8 q0, bf16x8 q1) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %3, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %4, 0"
      : "=&v"(s0), "=&v"(s1)
      : "v"(k), "a"(q0), "a"(q1));
}
__device__ __forceinline__ void mfma_result_fence_v(f32x4& r0, f32x4& r1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(r0), "+v"(r1));
}
__device__ __forceinline__ void mfma_result_fence_a(f32x4& r) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(r));
}
__device__ __forceinline__ void mfma_result_tie_a(f32x4& r) { asm volatile("" : "+a"(r)); }
// Hand-ordered building blocks for the FP8 inner loops.  Each is its own
// volatile asm statement, so the compiler keeps their relative order: MFMAs
// alternate with pairs of conversions and the conversions issue while the
// matrix core works.  Wait states: an MFMA that reads a register written by
// the VALU instruction just before it starts with s_nop 1 (the "_w" forms);
// elsewhere at least two instructions separate the two.  The compiler does
// not know the result latency of these MFMAs, so every group of them ends
// with a result fence on its accumulators before anything else touches them.
__device__ __forceinline__ uint32_t cvt_e4m3_lo(uint32_t w) {  // bytes 0, 1 -> bf16 x2
  uint32_t r;
  asm volatile("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  return r;
}
__device__ __forceinline__ uint32_t cvt_e4m3_hi(uint32_t w) {  // bytes 2, 3 -> bf16 x2
  uint32_t r;
  asm volatile("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
  return r;
}
// C (VGPR) += A (VGPR) * B (AGPR); the first of a chain starts from 0.
__device__ __forceinline__ void mfma_vva0_w(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_vva0(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_vva_w(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_vva(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
// C (VGPR) += A (VGPR) * B (VGPR); the "0" forms start a chain from 0.
__device__ __forceinline__ void mfma_vvv0_w(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vvv0(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vvv_w(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vvv(f32x4& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// Ends a group of hand-placed MFMAs: waits out the matrix pipe and the
// result latency while the last MFMAs' operands are still held, so that
// neither their source registers are reused nor their results read early.
#define MLA_O16(o) "+v"(o[0][0]), "+v"(o[0][1]), "+v"(o[0][2]), "+v"(o[0][3]), "+v"(o[0][4]), "+v"(o[0][5]), \
    "+v"(o[0][6]), "+v"(o[0][7]), "+v"(o[1][0]), "+v"(o[1][1]), "+v"(o[1][2]), "+v"(o[1][3]),            \
    "+v"(o[1][4]), "+v"(o[1][5]), "+v"(o[1][6]), "+v"(o[1][7])
__device__ __forceinline__ void mfma_drain_o(f32x4 (&o)[2][8], bf16x8 a0, bf16x8 a1, bf16x8 b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : MLA_O16(o) : "v"(a0), "v"(a1), "v"(b));
}
__device__ __forceinline__ void mfma_drain_s(f32x4& s0, f32x4& s1, bf16x8 a) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1) : "v"(a));
}
// The same hold without the wait: for the second half of a group whose first
// half's drain has already waited out the pipe.
__device__ __forceinline__ void mfma_tie_o(f32x4 (&o)[2][8], bf16x8 a0, bf16x8 a1, bf16x8 b) {
  asm volatile("" : MLA_O16(o) : "v"(a0), "v"(a1), "v"(b));
}
// Result fence alone on the sixteen P V accumulators.
__device__ __forceinline__ void mfma_result_fence_v16(f32x4 (&o)[2][8]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : MLA_O16(o));
}
// Zeroes the sixteen P V accumulators in place with MFMAs on zero operands,
// in one statement that also waits out their latency.  The compiler may
// materialise the zero operand with VALU moves right before the statement,
// so it starts with the wait states an MFMA needs after a VALU write of its
// source registers.
__device__ __forceinline__ void mfma_zero_o(f32x4 (&o)[2][8]) {
  const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %1, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %3, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %4, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %5, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %6, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %7, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %8, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %9, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %10, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %11, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %12, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %13, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %14, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %15, %16, %16, 0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
      : MLA_O16(o)
      : "v"(z));
}
// The same, defining the accumulators afresh (write-only operands): where the
// accumulators are zeroed at the top of a loop, no copy of their previous
// values has to be kept across the loop's back edge.
#define MLA_O16_DEF(o) "=&v"(o[0][0]), "=&v"(o[0][1]), "=&v"(o[0][2]), "=&v"(o[0][3]), "=&v"(o[0][4]), \
    "=&v"(o[0][5]), "=&v"(o[0][6]), "=&v"(o[0][7]), "=&v"(o[1][0]), "=&v"(o[1][1]), "=&v"(o[1][2]),      \
    "=&v"(o[1][3]), "=&v"(o[1][4]), "=&v"(o[1][5]), "=&v"(o[1][6]), "=&v"(o[1][7])
__device__ __forceinline__ void mfma_def_zero_o(f32x4 (&o)[2][8]) {
  const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %1, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %3, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %4, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %5, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %6, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %7, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %8, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %9, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %10, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %11, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %12, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %13, %16, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %14, %16, %16, 0\n\tv_mfma_f32_16x16x32_bf16 %15, %16, %16, 0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
      : MLA_O16_DEF(o)
      : "v"(z));
}
__device__ __forceinline__ bf16x8 bf16x8_of(const uint32_t (&d)[4]) {
  return __builtin_bit_cast(bf16x8, u32x4{d[0], d[1], d[2], d[3]});
}
// A value placed in AGPRs (a copy, once); later "a"-constrained uses keep it there.
__device__ __forceinline__ bf16x8 to_agpr(bf16x8 v) {
  bf16x8 r;
  asm volatile("" : "=a"(r) : "0"(v));
  return r;
}
// Orders readers of MFMA results after this point without waiting: for use
// where enough other instructions already separate them from the MFMAs.
__device__ __forceinline__ void mfma_result_tie_v(f32x4& r0, f32x4& r1) { asm volatile("" : "+v"(r0), "+v"(r1)); }
// A zero accumulator produced by an MFMA (zero operands, SrcC = 0): it gets
// the register class of the other MFMA accumulators it merges with, so no
// copies appear where a zeroed value and an accumulated one meet.
__device__ __forceinline__ f32x4 mfma_zero() {
  const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(z, z, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// 32 x 32 x 16 bf16 MFMAs on a 16-register accumulator (VGPRs), the same
// hand-placed conventions: "_w" forms wait out a VALU write of a source just
// before, "first" forms start a chain from 0, and the drain waits out the
// result latency while holding the last operands.
typedef __attribute__((ext_vector_type(16))) float f32x16;
__device__ __forceinline__ void mfma32_w(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_first(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_first_w(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_drain(f32x16& c0, f32x16& c1, bf16x8 a) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1) : "v"(a));
}
// Eight 32 x 32 accumulators ([2][4]) as one operand list: defined afresh by
// MFMAs on zero operands (the statement waits out their latency), tied to the
// last operands of a group of hand-placed MFMAs, or fenced before VALU reads.
#define MLA_O8_DEF(o) "=&v"(o[0][0]), "=&v"(o[0][1]), "=&v"(o[0][2]), "=&v"(o[0][3]), "=&v"(o[1][0]), \
    "=&v"(o[1][1]), "=&v"(o[1][2]), "=&v"(o[1][3])
#define MLA_O8(o) "+v"(o[0][0]), "+v"(o[0][1]), "+v"(o[0][2]), "+v"(o[0][3]), "+v"(o[1][0]), "+v"(o[1][1]), \
    "+v"(o[1][2]), "+v"(o[1][3])
__device__ __forceinline__ void mfma32_def_zero8(f32x16 (&o)[2][4]) {
  const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %8, %8, 0\n\tv_mfma_f32_32x32x16_bf16 %1, %8, %8, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %8, %8, 0\n\tv_mfma_f32_32x32x16_bf16 %3, %8, %8, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %8, %8, 0\n\tv_mfma_f32_32x32x16_bf16 %5, %8, %8, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %8, %8, 0\n\tv_mfma_f32_32x32x16_bf16 %7, %8, %8, 0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
      : MLA_O8_DEF(o)
      : "v"(z));
}
__device__ __forceinline__ void mfma32_tie8(f32x16 (&o)[2][4], bf16x8 a, bf16x8 b0, bf16x8 b1) {
  asm volatile("" : MLA_O8(o) : "v"(a), "v"(b0), "v"(b1));
}
__device__ __forceinline__ void mfma32_result_fence8(f32x16 (&o)[2][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : MLA_O8(o));
}
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace mla
