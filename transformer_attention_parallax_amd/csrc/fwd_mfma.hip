// fwd_mfma.hip -- Parallax attention prefill for bf16 inputs on the gfx950
// matrix cores.
//
// Parallax attention is softmax attention minus the key-value covariance
// contracted with a learned probe rho_i, evaluated over one shared pass of
// K and V for both branches (zubnet.ai news item on Parallax, second
// paragraph). Per query row the kernel accumulates
//     O_v  = sum_j p_ij v_j,        O_rv = sum_j p_ij r_ij v_j,
//     l    = sum_j p_ij,            R    = sum_j p_ij r_ij,
// with r_ij = rho_i . k_j and online-softmax weights p_ij, and writes
//     o_i = vbar + (vbar * rbar - O_rv / l),  vbar = O_v / l, rbar = R / l,
// which equals vbar - C_i rho_i (C_i the softmax-weighted value-key
// covariance).
//
// Four contractions per (query block, key tile), all on MFMA with fp32
// accumulation:
//   S^T  = K Q^T    and  Rk^T = K R^T    bf16 x bf16 (products exact in fp32)
//   O_v^T  += V^T P^T  and  O_rv^T += V^T (P o Rk)^T     fp16 x fp16
// The transposed forms put one query per lane column, so the per-query
// softmax state (max, l, R, rescale factor) is a per-lane scalar and row
// reductions need one exchange between the two lane halves. Each K fragment
// read from LDS feeds both S^T and Rk^T; each V^T fragment feeds both O_v^T
// and O_rv^T -- the matrix-core form of "both branches reuse one KV stream".
//
// Precision: p and p*r are fed to the second pair of contractions as fp16
// (11-bit significand; p in [0, 1], |p r| <= |r|), and V is converted from
// bf16 to fp16 once per tile (exact for |v| in [2^-14, 65504]). l and R are
// summed from the same fp16-rounded values the matrix cores consume, so the
// weights used for vbar and for the covariance term are the same numbers
// and the cancellation in vbar * rbar - O_rv / l stays benign. With bf16
// probabilities instead, the error on the large-probe 1.7B-model workload
// exceeds the 2e-2 budget.
//
// Tiling: 256 threads = 4 waves; a workgroup owns BM = 128 query rows of
// one (b, h), each wave 32 rows; key tiles of BN = 64 keys are staged in LDS
// (K row-major with a 16-byte row pad, V transposed to [D][BN] fp16 with an
// 8-byte pad) through a register prefetch of the next tile issued before
// the current tile's math. Causal: each wave skips the key tiles wholly
// above its own diagonal; the workgroups with the most tiles launch first.
// Lane layouts of v_mfma_f32_32x32x16_{bf16,f16} (checked on hardware):
//   A[i][k]: lane i + 32*(k/8), element k%8
//   B[k][j]: lane j + 32*(k/8), element k%8
//   C[i][j]: lane j + 32*((i/4)%2), register 4*(i/8) + i%4
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace parallax {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr int kWaveRows = 32;

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

__device__ __forceinline__ float finish(float inv, float rsum, float ov, float orv) {
#pragma clang fp contract(off)
  const float vbar = ov * inv;
  const float corr = vbar * (rsum * inv) - orv * inv;
  return vbar + corr;
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void fwd_mfma_kernel(FwdParams p) {
  constexpr int KSTR = D + 8;     // sK row stride (bf16 elements)
  constexpr int VSTR = kBN + 4;   // sVt row stride (fp16 elements)
  constexpr int DT = D / 16;      // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;      // 32-row blocks of O^T
  constexpr int NKB = kBN / 32;   // 32-key blocks per tile
  constexpr int CPR = D / 8;      // 16-byte chunks per K/V row
  constexpr int KPT = kBN * CPR / kThreads;  // tile rows loaded per thread
  static_assert(KPT == 2 || KPT == 4, "tile load split");

  __shared__ __attribute__((aligned(16))) unsigned short sK[kBN * KSTR];
  __shared__ __attribute__((aligned(16))) unsigned short sVt[D * VSTR];

  const int nqb = (p.N + kBM - 1) / kBM;
  // heavy (late) query blocks first under causal masking
  const int qb = p.causal ? (nqb - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lc = lane & 31;   // query column of this lane
  const int kg = lane >> 5;   // lane half
  const int q0 = qb * kBM;
  const int qw0 = q0 + wave * kWaveRows;  // first query of this wave
  const int qi = qw0 + lc;                // this lane's query
  const int N = p.N;

  // ---- this lane's Q and R fragments (B operand of S^T, Rk^T) --------------
  bf16x8_t qf[DT], rf[DT];
  {
    const char* qrow = reinterpret_cast<const char*>(p.q) +
                       (b * p.q_sb + (int64_t)qi * p.q_sn + h * p.q_sh) * 2;
    const char* rrow = reinterpret_cast<const char*>(p.rho) +
                       (b * p.r_sb + (int64_t)qi * p.r_sn + h * p.r_sh) * 2;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
      if (qi < N) {
        a = *reinterpret_cast<const u32x4*>(qrow + (16 * t + 8 * kg) * 2);
        c = *reinterpret_cast<const u32x4*>(rrow + (16 * t + 8 * kg) * 2);
      }
      qf[t] = __builtin_bit_cast(bf16x8_t, a);
      rf[t] = __builtin_bit_cast(bf16x8_t, c);
    }
  }

  // ---- tile loader: thread owns rows kq*KPT + i, 16-byte chunk dc ----------
  const int dc = tid % CPR;
  const int kq = tid / CPR;
  const char* kbase = reinterpret_cast<const char*>(p.k) +
                      (b * p.k_sb + h * p.k_sh + dc * 8) * 2;
  const char* vbase = reinterpret_cast<const char*>(p.v) +
                      (b * p.v_sb + h * p.v_sh + dc * 8) * 2;
  u32x4 kreg[KPT], vreg[KPT];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = j0 + kq * KPT + i;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kreg[i] = j < N ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)j * p.k_sn * 2) : z;
      vreg[i] = j < N ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)j * p.v_sn * 2) : z;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      *reinterpret_cast<u32x4*>(&sK[(kq * KPT + i) * KSTR + dc * 8]) = kreg[i];
    // V^T: column (key) run of KPT keys for each of the 8 d values
    unsigned hv[KPT][4];
#pragma unroll
    for (int i = 0; i < KPT; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) hv[i][w] = bf16x2_to_f16x2(vreg[i][w]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const bool hi = e & 1;
      unsigned short x[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        x[i] = hi ? (unsigned short)(hv[i][w] >> 16) : (unsigned short)(hv[i][w] & 0xffffu);
      unsigned short* dst = &sVt[(dc * 8 + e) * VSTR + kq * KPT];
      if constexpr (KPT == 4) {
        const u32x2 pr = {(unsigned)x[0] | ((unsigned)x[1] << 16),
                          (unsigned)x[2] | ((unsigned)x[3] << 16)};
        *reinterpret_cast<u32x2*>(dst) = pr;
      } else {
        *reinterpret_cast<unsigned*>(dst) = (unsigned)x[0] | ((unsigned)x[1] << 16);
      }
    }
  };

  // ---- accumulators ---------------------------------------------------------
  f32x16_t ov[DB], orv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) { ov[i][r] = 0.0f; orv[i][r] = 0.0f; }
  float m = -INFINITY;  // running max (base-2 units), same in both lane halves
  float lsum = 0.0f;    // this lane half's share of l
  float rsum = 0.0f;    // this lane half's share of R
  const float cs = p.scale_log2;

  int kend = N;
  if (p.causal) kend = (q0 + kBM < N) ? q0 + kBM : N;
  const int ntiles = (kend + kBN - 1) / kBN;
  const int wave_last_q = qw0 + kWaveRows - 1;

  load_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = it * kBN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < ntiles) load_tile(j0 + kBN);
    if (p.causal && j0 > wave_last_q) continue;  // tile wholly above diagonal
    if (qw0 >= N) continue;                      // rows past the sequence

    // ---- S^T and Rk^T for the NKB key blocks -------------------------------
    f32x16_t s[NKB], rk[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[kb][r] = 0.0f; rk[kb][r] = 0.0f; }
      const unsigned short* krow = &sK[(kb * 32 + lc) * KSTR + 8 * kg];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(krow + 16 * t);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[kb], 0, 0, 0);
        rk[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, rf[t], rk[kb], 0, 0, 0);
      }
    }

    // ---- online softmax on this lane's 2*16 keys ---------------------------
    // key of (kb, r) for this lane: j0 + 32*kb + 8*(r/4) + 4*kg + r%4
    const bool need_mask = (p.causal && j0 + kBN - 1 > qw0) || (j0 + kBN > N);
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r] * cs;
        if (need_mask) {
          const int kj = j0 + 32 * kb + 8 * (r >> 2) + 4 * kg + (r & 3);
          if (kj >= N || (p.causal && kj > qi)) x = -INFINITY;
        }
        s[kb][r] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(m, mloc);
    const float alpha = (mnew == m) ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);
    const bool live = mnew != -INFINITY;
    m = mnew;

    f16x8_t pf[NKB][2], prf[NKB][2];
    float ls = 0.0f, rs = 0.0f;
    const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int r = 8 * hf + e;
          const float p0 = live ? __builtin_amdgcn_exp2f(s[kb][r] - mnew) : 0.0f;
          const float p1 = live ? __builtin_amdgcn_exp2f(s[kb][r + 1] - mnew) : 0.0f;
          const f32x2_t pp = {p0, p1};
          const f32x2_t qq = {p0 * rk[kb][r], p1 * rk[kb][r + 1]};
          const f16x2_t ph = __builtin_convertvector(pp, f16x2_t);
          const f16x2_t qh = __builtin_convertvector(qq, f16x2_t);
          ls = __builtin_amdgcn_fdot2(ph, one2, ls, false);
          rs = __builtin_amdgcn_fdot2(qh, one2, rs, false);
          pf[kb][hf][e] = ph[0];
          pf[kb][hf][e + 1] = ph[1];
          prf[kb][hf][e] = qh[0];
          prf[kb][hf][e + 1] = qh[1];
        }
    lsum = fmaf(lsum, alpha, ls);
    rsum = fmaf(rsum, alpha, rs);
    if (alpha != 1.0f) {
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) { ov[i][r] *= alpha; orv[i][r] *= alpha; }
    }

    // ---- O_v^T += V^T P^T,  O_rv^T += V^T (P o Rk)^T ------------------------
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key0 = 32 * kb + 16 * hf + 4 * kg;
#pragma unroll
        for (int i = 0; i < DB; ++i) {
          const unsigned short* vrow = &sVt[(32 * i + lc) * VSTR + key0];
          const f16x4_t lo = *reinterpret_cast<const f16x4_t*>(vrow);
          const f16x4_t hi = *reinterpret_cast<const f16x4_t*>(vrow + 8);
          const f16x8_t vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          ov[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kb][hf], ov[i], 0, 0, 0);
          orv[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, prf[kb][hf], orv[i], 0, 0, 0);
        }
      }
  }

  // ---- epilogue -------------------------------------------------------------
  const float l = lsum + __shfl_xor(lsum, 32);
  const float R = rsum + __shfl_xor(rsum, 32);
  if (qi < N) {
    const bool any = l > 0.0f;
    const float inv = any ? 1.0f / l : 0.0f;
    const int64_t obase = b * p.o_sb + (int64_t)qi * p.o_sn + h * p.o_sh;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * i + 8 * g + 4 * kg;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = any ? finish(inv, R, ov[i][4 * g + e], orv[i][4 * g + e]) : 0.0f;
        if constexpr (OUT_BF16) {
          unsigned short* dst = reinterpret_cast<unsigned short*>(p.out) + obase + d;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = f32_to_bf16_bits(o[e]);
        } else {
          float* dst = reinterpret_cast<float*>(p.out) + obase + d;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[e] = o[e];
        }
      }
  }
}

template <int D>
hipError_t launch_mfma(const FwdParams& p, bool out_bf16, hipStream_t stream) {
  const dim3 grid((p.N + kBM - 1) / kBM, p.H, p.B);
  if (out_bf16)
    hipLaunchKernelGGL((fwd_mfma_kernel<D, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<D, false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int D, bool out_bf16,
                           hipStream_t stream) {
  return D == 128 ? launch_mfma<128>(p, out_bf16, stream)
                  : launch_mfma<64>(p, out_bf16, stream);
}

}  // namespace parallax
