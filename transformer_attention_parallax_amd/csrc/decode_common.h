// decode_common.h -- device helpers shared by the decode kernels
// (decode.hip, decode_gqa.hip): wave64 group reductions over the lanes that
// hold one key row, 16-byte streaming loads, bf16 dot products and the
// per-element output formula of Parallax attention.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace parallax {
namespace dec {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float bf16_lo(unsigned w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(unsigned w) {
  return __uint_as_float(w & 0xffff0000u);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPK lanes. Every step pairs lanes
// symmetrically, so all lanes of a group end with bitwise-equal sums.
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<0xB1>(x);                      // quad_perm(1,0,3,2)
  x += dpp_f32<0x4E>(x);                      // quad_perm(2,3,0,1)
  if constexpr (LPK >= 8) x += dpp_f32<0x141>(x);   // row_half_mirror
  if constexpr (LPK >= 16) x += dpp_f32<0x140>(x);  // row_mirror
  if constexpr (LPK >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Dot product of eight bf16 pairs (two packed per dword), fp32 accumulate.
__device__ __forceinline__ float dot_bf16(const u32x4& a, const u32x4& b) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // copy the lane element out first: a bit cast taken directly on a
    // vector-element lvalue reads element 0
    const unsigned ai = a[i], bi = b[i];
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ai),
                                        __builtin_bit_cast(bf16x2_t, bi), s, false);
  }
  return s;
}

__device__ __forceinline__ void unpack_bf16(const u32x4& w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float x) {
  if constexpr (OUT_BF16)
    reinterpret_cast<unsigned short*>(base)[idx] = f32_to_bf16_bits(x);
  else
    reinterpret_cast<float*>(base)[idx] = x;
}

// Finish one output element from merged sums:
//   o = vbar + (vbar * rbar - A_rv / l).
// Products are rounded separately (no contraction), so a single visible key
// gives vbar * rbar == A_rv / l bit for bit and o == v exactly.
__device__ __forceinline__ float finish(float l, float ar, float av, float arv) {
#pragma clang fp contract(off)
  if (!(l > 0.0f)) return 0.0f;
  const float inv = 1.0f / l;
  const float vbar = av * inv;
  const float corr = vbar * (ar * inv) - arv * inv;
  return vbar + corr;
}

}  // namespace dec
}  // namespace parallax
