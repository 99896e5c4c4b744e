// proj.hip -- the fused input projection of a Parallax layer: one bf16
// product y = x W^T with W = [W_Q; W_K; W_V; W_R] stacked along the output
// features, so the probe rho = W_R x (zubnet.ai news item on Parallax,
// second paragraph: a learned projection of the layer input) comes out of
// the same pass over x as q, k and v. Each quarter of a row of y, viewed as
// [H, D], is directly a strided input of the attention kernels.
//
// C[M, N] = A[M, K] B[N, K]^T, bf16 operands, fp32 accumulation, bf16 (RNE)
// output. M = tokens (any), N = output features (multiple of 256), K = input
// features (multiple of 64).
//
// Workgroup: 256 x 256 outputs, 8 waves as 2 (M) x 4 (N), each 128 x 64 =
// 8 x 4 products v_mfma_f32_16x16x32_bf16 per 32-wide k step. K advances in
// steps of 64 through two LDS stages of A and B tiles (2 x 64 KiB), filled by
// buffer loads that write LDS directly; the next step's loads are in flight
// while the current step is consumed. Tile rows are 128 bytes (8 chunks of
// 16); chunk c of row r sits at slot c ^ ((r >> 1) & 7), so the 16 rows one
// fragment load touches fall in 16 distinct bank groups. Operand layouts
// (lane = c + 16 g): A fragment lane (i, g) holds A[i][8g .. 8g+7] of a
// 16 x 32 block, B likewise for a row of B, and the 16 x 16 result holds
// C[4g + r][c] in register r.
//
// Block order: workgroup i runs on XCD i % 8; each XCD takes a contiguous
// range of blocks, walked in groups of 8 M-blocks by all N-blocks (M
// fastest), so the 32 blocks an XCD runs at once share 8 A and 4 B slices of
// each k step in its L2.
#include "internal.h"
#include "mfma_common.h"

namespace parallax {
namespace {

using namespace mfma;

constexpr int kPM = 256;      // block rows (tokens)
constexpr int kPN = 256;      // block columns (output features)
constexpr int kPK = 64;       // k step
constexpr int kPW = 8;        // waves
constexpr int kGroupM = 8;    // M-blocks per ordering group

__device__ __forceinline__ void pdma16(__amdgpu_buffer_rsrc_t r, unsigned short* dst,
                                       int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ int pswz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(64 * kPW) void proj_kernel(ProjParams p) {
  constexpr int TILE = kPM * kPK;        // elements of one A (or B) stage
  constexpr int IPW = TILE * 2 / 1024 / kPW;  // 1-KiB loads per wave per tile: 4
  __shared__ __attribute__((aligned(1024))) unsigned short smem[2 * 2 * TILE];

  // ---- block order ---------------------------------------------------------
  const int nbm = (p.M + kPM - 1) / kPM;
  const int nbn = p.N / kPN;
  const int total = nbm * nbn;
  const int id = (int)blockIdx.x;
  const int lin = (total & 7) == 0 ? (id & 7) * (total >> 3) + (id >> 3) : id;
  const int per_group = kGroupM * nbn;
  const int group = lin / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, nbm - first_m);
  const int within = lin - group * per_group;
  const int mb = first_m + within % gm;
  const int nb = within / gm;
  const int m0 = mb * kPM;
  const int n0 = nb * kPN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int wm = wave >> 2;              // 128-row half
  const int wn = wave & 3;               // 64-column quarter

  // ---- staging: load ii of this wave covers tile rows 8 ii .. 8 ii + 7 ------
  const char* abase = reinterpret_cast<const char*>(p.x) + (int64_t)m0 * p.x_st * 2;
  const char* bbase = reinterpret_cast<const char*>(p.w) + (int64_t)n0 * p.w_st * 2;
  const int rows_a = min(kPM, p.M - m0);
  const int arec = (rows_a - 1) * (int)p.x_st * 2 + p.K * 2;   // rows past M read 0
  const int brec = (kPN - 1) * (int)p.w_st * 2 + p.K * 2;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase, arec);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bbase, brec);
  int aoff[IPW], boff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (IPW * wave + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ pswz(r);
    aoff[i] = r * (int)p.x_st * 2 + c * 16;
    boff[i] = r * (int)p.w_st * 2 + c * 16;
  }
  auto issue = [&](int kstep, int stage) {
    unsigned short* sa = smem + stage * 2 * TILE;
    unsigned short* sb = sa + TILE;
    const int kb = kstep * kPK * 2;
#pragma unroll
    for (int i = 0; i < IPW; ++i) pdma16(ra, sa + (IPW * wave + i) * 512, aoff[i] + kb);
#pragma unroll
    for (int i = 0; i < IPW; ++i) pdma16(rb, sb + (IPW * wave + i) * 512, boff[i] + kb);
  };

  // fragment offsets (elements within a stage's tile): row, then chunk slot
  int afo[8][2], bfo[4][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const int r = wm * 128 + mt * 16 + lc;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) afo[mt][ks] = r * kPK + (((4 * ks + lg) ^ pswz(r)) << 3);
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int r = wn * 64 + nt * 16 + lc;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) bfo[nt][ks] = r * kPK + (((4 * ks + lg) ^ pswz(r)) << 3);
  }

  f32x4_t acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = p.K / kPK;
  issue(0, 0);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    if (t + 1 < nk) issue(t + 1, (t + 1) & 1);
    const unsigned short* sa = smem + (t & 1) * 2 * TILE;
    const unsigned short* sb = sa + TILE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t bf[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        bf[nt] = *reinterpret_cast<const bf16x8_t*>(sb + bfo[nt][ks]);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(sa + afo[mt][ks]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[nt], acc[mt][nt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: bf16 through LDS, 16-byte row stores ----------------------
  // wave region: 128 rows x 64 columns, row stride 64 elements
  unsigned short* so = smem + wave * (128 * 64);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        so[(mt * 16 + 4 * lg + r) * 64 + nt * 16 + lc] = f32_to_bf16_bits(acc[mt][nt][r]);
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  unsigned short* y = reinterpret_cast<unsigned short*>(p.y);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = i * 8 + (lane >> 3);           // row within the wave region
    const int c = (lane & 7) * 8;                // first of 8 columns
    const int m = m0 + wm * 128 + r;
    const u32x4 v = *reinterpret_cast<const u32x4*>(so + r * 64 + c);
    if (m < p.M)
      *reinterpret_cast<u32x4*>(y + (int64_t)m * p.y_st + n0 + wn * 64 + c) = v;
  }
}

}  // namespace

hipError_t launch_proj(const ProjParams& p, hipStream_t stream) {
  const int nbm = (p.M + kPM - 1) / kPM;
  const int blocks = nbm * (p.N / kPN);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(proj_kernel, dim3(blocks), dim3(64 * kPW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace parallax
