// Device-side building blocks shared by the LAGA kernels (gfx950 / CDNA4).
//
// Matrix-core atoms: every contraction in this library is expressed with the
// 32x32 MFMA family.  For an atom with KPL elements per lane, lane l of a
// 64-wide wavefront supplies
//   A operand: row (l % 32), k = (l / 32) * KPL + [0, KPL)
//   B operand: col (l % 32), k = (l / 32) * KPL + [0, KPL)
// and receives 16 fp32 results at
//   C[r]: row 8 * (r / 4) + 4 * (l / 32) + (r % 4), col (l % 32),  r in [0, 16).
// One instruction covers K = 2 * KPL.  Because A and B use the same k
// assignment, any consistent permutation of k between the two operands gives
// the same dot products; the attention kernels use that to feed accumulator
// registers straight back in as the next contraction's operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "laga.h"

namespace laga {

typedef _Float16 half_t;
typedef uint16_t bf16_t;  // raw bfloat16 bit pattern
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bfx8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {  // round to nearest even (hardware conversion)
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Element tags for templated code: what a value is stored as in memory.
struct Bf16In {};  // raw bfloat16 bits
struct F32In {};   // float32

template <class Tag> struct InType;
template <> struct InType<Bf16In> { typedef bf16_t type; static constexpr int bytes = 2; };
template <> struct InType<F32In> { typedef float type; static constexpr int bytes = 4; };

__device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(half_t v) { return static_cast<float>(v); }

// ------------------------------------------------------------ MFMA element types
// Matrix-core operand types: fp16, bf16 (stored as raw bits in LDS) and fp32.
struct MmaF16 {
  typedef half_t elem;
  typedef half8 frag;
  static constexpr int KPL = 8;
  static constexpr int K = 16;
  __device__ static __forceinline__ elem from_f32(float f) { return static_cast<half_t>(f); }
  __device__ static __forceinline__ float to_f32(elem e) { return static_cast<float>(e); }
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

struct MmaBf16 {
  typedef bf16_t elem;
  typedef u16x8 frag;
  static constexpr int KPL = 8;
  static constexpr int K = 16;
  __device__ static __forceinline__ elem from_f32(float f) { return f32_to_bf16(f); }
  __device__ static __forceinline__ float to_f32(elem e) { return bf16_to_f32(e); }
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bfx8, a),
                                                   __builtin_bit_cast(bfx8, b), c, 0, 0, 0);
  }
};

struct MmaF32 {
  typedef float elem;
  typedef float frag;
  static constexpr int KPL = 1;
  static constexpr int K = 2;
  __device__ static __forceinline__ elem from_f32(float f) { return f; }
  __device__ static __forceinline__ float to_f32(elem e) { return e; }
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// ------------------------------------------------------------ fp8 (OCP e4m3)
// The low part of a split K/V value (x - fp16(x), at most 2^-11 |x|) is kept
// as e4m3 bytes scaled by 2^kLoShift: with |x| < 256 the scaled value stays
// below e4m3's 448, and the 3-bit mantissa leaves x represented to ~2^-15.
// Larger |x| saturate the low byte, which degrades gracefully towards fp16.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int kLoShift = LAGA_KV_LO_SHIFT;
constexpr float kE4m3Max = 448.f;

// Four floats -> four e4m3 bytes, first value in the lowest byte (round to
// nearest even; saturated at +-448 before conversion).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  b = fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
  c = fminf(fmaxf(c, -kE4m3Max), kE4m3Max);
  d = fminf(fmaxf(d, -kE4m3Max), kE4m3Max);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// The same for values already within +-448 (no saturation step).
__device__ __forceinline__ uint32_t pack_e4m3x4_in_range(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// Power-of-two shift s for a row of e4m3 values with largest magnitude m:
// m * 2^s lies in [128, 256) (below e4m3's 448 with room for rounding); 0 for
// an all-zero row.  Clamped so that 127 - s stays a valid E8M0 scale byte.
__device__ __forceinline__ int e4m3_row_shift(float m) {
  const int e = static_cast<int>((__float_as_uint(m) >> 23) & 0xff);  // m = 1.f * 2^(e - 127)
  if (e == 0) return 0;
  const int s = 134 - e;  // 2^(e - 127) * 2^s = 2^7
  return s < -120 ? -120 : (s > 120 ? 120 : s);
}

// Bytes 2*HI .. 2*HI+1 of w (e4m3) -> two floats.
template <bool HI>
__device__ __forceinline__ f32x2 unpack_e4m3x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
}

// C += (A * 2^(ea-127)) . (B * 2^(eb-127)) with e4m3 operands, K = 64: lane l
// supplies row / column l % 32 and k = (l / 32) * 32 + [0, 32) as 32 bytes.
// The scales act per row of A / column of B: lanes l and l ^ 32 must pass the
// same ea (eb) -- with different values the products came out wrong, as if
// one lane's scale were applied to both halves of k.
__device__ __forceinline__ f32x16 mma_e4m3(i32x8 a, i32x8 b, f32x16 c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// Split a float into NS terms of the MMA element type: x ~= sum_s part[s].
template <class M, int NS>
__device__ __forceinline__ void split_to(float x, typename M::elem* part) {
  float r = x;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    part[s] = M::from_f32(r);
    r -= M::to_f32(part[s]);
  }
}

// fp16 hi/lo pairs of x0 and x1: hi = fp16(x) and lo = fp16(x - hi), both
// rounded to nearest even, as split_to<fp16, 2> gives them.  x - hi is exact
// in fp32, so one mixed-precision FMA per value forms and rounds it, and one
// packed conversion makes both hi terms.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_f16_pair(float x0, float x1, half2_t& hi, half2_t& lo) {
  hi = __builtin_convertvector(f32x2{x0, x1}, half2_t);
  // (The compiler turns the FMA form back into a convert and a subtract
  // about half the time; the two VALU instructions are therefore stated.)
  const uint32_t h = __builtin_bit_cast(uint32_t, hi);
  uint32_t l;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l) : "v"(h), "v"(x0));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(l) : "v"(h), "v"(x1));
  lo = __builtin_bit_cast(half2_t, l);
}

// bf16 hi/lo pairs of x0 and x1 (hi = bf16(x), lo = bf16(x - hi), both
// rounded to nearest even, as split_to<bf16, 2> gives them), packed two to a
// word: one packed conversion per pair and term, x - hi exact in fp32.
__device__ __forceinline__ void split_bf16_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2_t));
  const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2_t));
}

// Load a KPL-element fragment from LDS (contiguous, aligned to KPL elements).
template <class M>
__device__ __forceinline__ typename M::frag lds_frag(const typename M::elem* p) {
  return *reinterpret_cast<const typename M::frag*>(p);
}

// ------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Exchange with the lane 32 positions away (the other half of the wavefront).
__device__ __forceinline__ float swap_halves(float v) { return __shfl_xor(v, 32, kWave); }

// max / sum of v over lanes l and l ^ 32, in every lane, without LDS: gfx950's
// v_permlane32_swap given (v, v) returns the lower half duplicated in one
// result and the upper half duplicated in the other.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of key `k` (0..BN-1) inside an LDS row that a 32x32 atom reads as a
// K-operand fed from accumulator registers: bits 2 and 3 of the key index are
// swapped, so that the KPL keys one lane needs for one MFMA step are contiguous.
__device__ __forceinline__ int acc_key_col(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

}  // namespace laga
