// mfma_common.h -- device helpers shared by the bf16 prefill kernels:
// vector types, bf16 <-> fp16 conversion, buffer-resource loads, cross-lane
// exchanges and the per-row output formula of Parallax attention.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace parallax {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kBN = 64;             // keys per staged tile
constexpr float kTau = 8.0f;        // headroom (base-2) before a rescale
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, gfx9 data format

// Layout of a row-major bf16 tile [rows][D] in LDS that is read both as
// 16-row MFMA fragments (ds_read_b128: lane (i, g) reads row i, 16-byte
// chunk 4 t + tile_chunk<D>(g) of the head dimension) and through the
// transposing LDS read (ds_read_b64_tr_b16: 32 lanes read two adjacent
// chunks of 8 rows). On gfx950 a 16-byte read is served 16 lanes at a time,
// the low half (i < 8) of one lane group with the high half of its
// neighbour, and a transposing read 32 lanes at a time (measured with the
// LDS bank-conflict counter). Chunk c of row r sits at slot
// c ^ tile_swz<D>(r). For D = 128 (16 slots per 256-byte row) the 4-bit
// row index is rotated by one, so rows 0..7 take even and rows 8..15 odd
// values, and neighbouring lane groups take chunks two apart; then both
// kinds of pass touch 16 distinct 16-byte bank groups. For D = 64 (8 slots
// per 128-byte row) r % 8 with the natural chunk order already does. Both
// depend on r % 16 only, so row offsets of 16 are immediates.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  const int x = r & 15;
  return D == 128 ? (((x << 1) | (x >> 3)) & 15) : (x & 7);
}
// Head-dimension chunk (within each group of four) lane group g supplies to
// a contraction over D; the same order must be used for both operands.
template <int D>
__device__ __forceinline__ int tile_chunk(int g) {
  return D == 128 ? (((g & 1) << 1) | (g >> 1)) : g;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// Two bf16 (packed in one dword) -> two fp16 (packed), via fp32.
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned w) {
  const f32x2_t x = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(x, f16x2_t));
}

// o = vbar + (vbar * rbar - O_rv / l) with vbar = O_v / l, rbar = R / l;
// evaluated in this order, without contraction, on every path.
__device__ __forceinline__ float finish(float inv, float rsum, float ov, float orv) {
#pragma clang fp contract(off)
  const float vbar = ov * inv;
  const float corr = vbar * (rsum * inv) - orv * inv;
  return vbar + corr;
}

// Buffer resource over [base, base + bytes); loads at or past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base,
                                                           int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, n,
                                           kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// x from lane ^ 16 (within each 32-lane half) and from lane ^ 32.
__device__ __forceinline__ float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
__device__ __forceinline__ float xor32(float x, int bperm_addr) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(bperm_addr, __float_as_int(x)));
}

}  // namespace mfma
}  // namespace parallax
