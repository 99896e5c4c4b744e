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
  // Grouped-query / paged decode (decode_gqa.hip); H above is the number
  // of query heads, Hkv = H / group the number of key-value heads.
  int Hkv;
  const int32_t* block_table;  // nullable: [B] rows of page indices
  int64_t bt_sb;               // row stride of block_table
  int page;                    // tokens per page (multiple of 8)
  int num_pages;               // pages in the cache; other indices are skipped
  // Workgroup shape of the grouped kernel: gqa_nh kv heads of one sequence
  // per workgroup, gqa_wph waves per kv head (gqa_nh * gqa_wph <= 8 waves;
  // gqa_nh divides Hkv).
  int gqa_nh, gqa_wph;
  // Query rows as streams (fp32 inputs only; decode.hip): with rows > 0,
  // stream z of the grid is query row z % rows of sequence z / rows, its
  // q, rho and out rows at the row strides below, and it sees keys
  // [0, row + 1) when causal_rows is set, else [0, Lmax); seqlens unused,
  // nsplit = 1.
  int rows;
  int causal_rows;
  int64_t q_sn, r_sn, o_sn;
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
  // Packed sequences (nullable): sequence b is rows [cu_seqlens[b],
  // cu_seqlens[b+1]) of each tensor along n (the b strides are unused) and
  // N is the longest length; without it every sequence has N rows.
  const int32_t* cu_seqlens;
  // Training forward (nullable): also write vbar [B][N][H][D] fp32 and per
  // query {lse2, rbar} to lse_rbar [B][H][N] float2 (dense batches only).
  float* vbar;
  float* lse_rbar;
};

// fp16 elements of one packed V^T key tile (64 keys x D).
inline constexpr int fwd_tile_elems(int D) { return 64 * D; }

// Floats per split record: m, l, A_r, pad, A_v[D], A_rv[D].
inline constexpr int decode_record_floats(int D) { return 4 + 2 * D; }

// Most key ranges one decode call may be split into.
inline constexpr int kMaxDecodeSplits = 1024;

// Transposed tile images of a [B, N, H, D] bf16 tensor (pack.hip).
struct PackParams {
  const void* src;
  int64_t sb, sn, sh;      // element strides of src
  int B, N, H;
  void* dst;               // [B][H][tiles][D][T] 16-bit elements
  int tiles;               // ceil(N / T)
  const int32_t* cu_seqlens;  // nullable: packed sequences, as in FwdParams
};

// Backward of the bf16 prefill (bwd_mfma.hip). Inputs bf16 [B, N, H, D]
// with (b, n, h) element strides; gradients fp32 with their own strides.
struct BwdParams {
  const void *q, *k, *v, *rho, *dout;
  int64_t q_sb, q_sn, q_sh, k_sb, k_sn, k_sh, v_sb, v_sn, v_sh;
  int64_t r_sb, r_sn, r_sh, g_sb, g_sn, g_sh;
  float *dq, *dk, *dv, *drho;
  int64_t dq_sb, dq_sn, dq_sh, dk_sb, dk_sn, dk_sh;
  int64_t dv_sb, dv_sn, dv_sh, dr_sb, dr_sn, dr_sh;
  int B, N, H;
  int causal;
  float scale;             // softmax scale
  float scale_log2;        // softmax scale * log2(e)
  const float* stats;      // [B][H][N] float4 from the statistics pass
  // Backward from a training forward's saved tensors (saved_out non-null):
  // the query-block kernel forms each query's statistics itself from the
  // saved o (fp32 or bf16, strides so_*), vbar [B][N][H][D] fp32 and
  // {lse2, rbar} [B][H][N] float2, and writes them to stats_w (= stats)
  // for the key-block kernel that follows.
  const void* saved_out;
  int64_t so_sb, so_sn, so_sh;
  int saved_out_bf16;
  const float* saved_vbar;
  const float* saved_lse_rbar;
  float* stats_w;
};

// Fused input projection y = x W^T (proj.hip): bf16, element strides of rows.
struct ProjParams {
  const void* x;     // [M, K]
  int64_t x_st;
  const void* w;     // [N, K]
  int64_t w_st;
  void* y;           // [M, N] bf16
  int64_t y_st;
  int M, N, K;
};

// Launchers return the hipError_t of the launch.
hipError_t launch_pack_t(const PackParams& p, int D, int T, bool to_f16,
                         hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int D, bool in_bf16,
                         bool out_bf16, hipStream_t stream);
// Merge of the split records written by either decode kernel (decode.hip).
hipError_t launch_decode_combine(const DecodeParams& p, int D, bool out_bf16,
                                 hipStream_t stream);
// Grouped-query, optionally paged decode, bf16 inputs (decode_gqa.hip).
hipError_t launch_decode_gqa(const DecodeParams& p, int D, int group,
                             bool out_bf16, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int D, bool out_bf16,
                          hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdParams& p, int D, bool out_bf16,
                           hipStream_t stream);
hipError_t launch_proj(const ProjParams& p, hipStream_t stream);
// Streaming read of [src, src + bytes) XOR-folded into *sink (stream.hip).
hipError_t launch_stream_read(const void* src, int64_t bytes, unsigned* sink,
                              hipStream_t stream);
// dq, drho (per query block) then dk, dv (per key block).
hipError_t launch_bwd_bf16(const BwdParams& p, int D, hipStream_t stream);
// Statistics pass of the backward: per query {lse2, 1 + rbar, g.vbar,
// g.o + rbar g.vbar} to p.stats_w [B][H][N] float4.
hipError_t launch_bwd_stats_bf16(const BwdParams& p, int D, hipStream_t stream);

}  // namespace parallax
