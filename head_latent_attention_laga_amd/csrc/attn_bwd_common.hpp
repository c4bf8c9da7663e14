// Pieces shared by the two attention-backward kernels (dK/dV and dq): the
// argument block and staging helpers.
#pragma once

#include <type_traits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace laga {
namespace bwd {

constexpr int kThreads = 256;  // 4 wavefronts, one per SIMD
constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
  const void* q; const void* k_nope; const void* k_pe; const void* v;
  const float* lse; const float* delta; const void* d_o;
  void* dkv; float* dk_pe_part; float* dq;
  // e4m3 q_nope / dO rows and their E8M0 row scales (split operands, dK/dV).
  const uint8_t* q8; const uint8_t* do8; const int* qsc; const int* osc;
  // dO (and with it delta, dP, dS) enters scaled by 2^g, g = *do_shift
  // (nullptr: g = 0); the kernels scale their outputs by 2^-g.
  const int* do_shift;
  int64_t S, plane_k, plane_v, plane_dkv; int B, h; float scale_log2, scale;
};

// 16-byte chunk of `E` converted from a 16-byte chunk of the input type.
template <class E, class InT>
__device__ __forceinline__ void convert_chunk(u32x4 raw, E* out) {
  if constexpr (std::is_same<InT, E>::value) {  // same type
    *reinterpret_cast<u32x4*>(out) = raw;
  } else if constexpr (std::is_same<InT, bf16_t>::value && std::is_same<E, half_t>::value) {  // bf16 -> fp16
    const u16x8 v = __builtin_bit_cast(u16x8, raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = static_cast<E>(bf16_to_f32(v[j]));
  } else {
    static_assert(std::is_same<InT, E>::value, "unsupported conversion");
  }
}

// 2^g and 2^-g for the dO scale (g = 0 without one).
__device__ __forceinline__ int do_shift_of(const BwdArgs& a) {
  return a.do_shift ? __builtin_amdgcn_readfirstlane(*a.do_shift) : 0;
}
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float(static_cast<uint32_t>(127 + e) << 23); }

template <class T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const T* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, bytes, 0x00020000);
}


inline BwdArgs make_args(const Shape& s, const void* q, const void* kn, const void* kp, const void* v, const float* lse,
                  const float* delta, const void* d_o) {
  BwdArgs a;
  a.q = q; a.k_nope = kn; a.k_pe = kp; a.v = v; a.lse = lse; a.delta = delta; a.d_o = d_o;
  a.dkv = nullptr; a.dk_pe_part = nullptr; a.dq = nullptr;
  a.q8 = nullptr; a.do8 = nullptr; a.qsc = nullptr; a.osc = nullptr; a.do_shift = nullptr;
  a.S = s.S; a.B = static_cast<int>(s.B); a.h = s.h;
  a.plane_k = s.T * s.h * s.d_nope;
  a.plane_v = s.T * s.h * s.d_v;
  a.plane_dkv = s.T * s.h * s.C();
  a.scale = 1.0f / sqrtf(static_cast<float>(s.d_qk()));
  a.scale_log2 = kLog2e * a.scale;
  return a;
}


}  // namespace bwd
}  // namespace laga
