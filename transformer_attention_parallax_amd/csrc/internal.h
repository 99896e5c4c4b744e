// internal.h -- parameter blocks and launchers shared by the C ABI layer
// (api.hip) and the kernels. Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace parallax {

// One decode problem, already validated. Strides in elements.
struct DecodeParams {
  const void* q;
  const void* rho;
  const void* k;
  const void* v;
  const int32_t* seqlens;  // nullable
  void* out;
  float* ws;               // [B, H, nsplit, rec] fp32 partial records
  int64_t q_sb, q_sh, r_sb, r_sh;
  int64_t kv_sb, kv_sh, kv_sl;
  int64_t o_sb, o_sh;
  int B, H, Lmax;
  int nsplit;              // >= 1
  int chunk;               // keys per split
  float scale_log2;        // softmax scale * log2(e)
};

// One prefill problem, already validated. Strides in elements.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* rho;
  void* out;
  int64_t q_sb, q_sn, q_sh;
  int64_t k_sb, k_sn, k_sh;
  int64_t v_sb, v_sn, v_sh;
  int64_t r_sb, r_sn, r_sh;
  int64_t o_sb, o_sn, o_sh;
  int B, N, H;
  int causal;
  float scale_log2;        // softmax scale * log2(e)
  unsigned short* vt;      // bf16 path: workspace for the fp16 V^T tiles
  int vt_tiles;            // key tiles per (b, h) in vt: ceil(N / 64)
};

// fp16 elements of one packed V^T key tile (64 keys x D).
inline constexpr int fwd_tile_elems(int D) { return 64 * D; }

// Floats per split record: m, l, A_r, pad, A_v[D], A_rv[D].
inline constexpr int decode_record_floats(int D) { return 4 + 2 * D; }

// Launchers return the hipError_t of the launch.
hipError_t launch_decode(const DecodeParams& p, int D, bool in_bf16,
                         bool out_bf16, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int D, bool out_bf16,
                          hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdParams& p, int D, bool out_bf16,
                           hipStream_t stream);

}  // namespace parallax
