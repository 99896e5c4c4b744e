// fwd_valu.hip -- Parallax attention prefill on the vector ALUs (fp32 math).
//
// A tiled fp32-input path: q, k, v, rho in fp32, every product and sum in
// fp32. The library runs fp32 prefill as one decode stream per query row
// (decode.hip, rows mode) wherever that applies, which is faster at every
// size measured; this kernel serves the calls it cannot take (K and V with
// different strides, more than 65535 rows). It is a tiled flash-style kernel: one 256-thread workgroup owns
// BM query rows of one (b, h) and walks key tiles of BN keys, keeping per
// row the online-softmax state (m, l, A_r) and the two D-wide accumulators
// A_v = sum p v and A_rv = sum p r v, r = rho . k (one pass over K and V for
// both branches, as the zubnet.ai news item on Parallax describes in its
// second paragraph). The output is o = vbar (1 + rbar) - A_rv / l, i.e.
// softmax attention minus the value-key covariance contracted with rho.
//
// Thread layout: 8 threads per query row (32 rows x 8 = 256). In the score
// phase thread (i, c) computes keys c, c+8, ... of the key tile (32 keys at
// D = 64, 16 at D = 128); in the accumulate phase it owns output columns
// c, c+8, ... of row i. Row reductions use 8-lane shuffles. Tiles live in
// LDS with a one-float row pad so that the eight distinct rows (or columns)
// touched by a wave fall in distinct banks. The next key and value tile is
// loaded into registers (16-byte loads) while the current one is computed,
// then stored to LDS behind a barrier, so each tile's global-memory latency
// overlaps the previous tile's arithmetic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace parallax {
namespace {

constexpr int kBM = 32;
constexpr int kBN = 16;
constexpr int kThreads = 256;
constexpr int kTPR = 8;  // threads per row

__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (BF16)
    return __uint_as_float((unsigned)reinterpret_cast<const unsigned short*>(base)[idx] << 16);
  else
    return reinterpret_cast<const float*>(base)[idx];
}

// o = vbar + (vbar * rbar - A_rv / l) with separately rounded products, so
// that a row with one visible key returns that key's value exactly.
__device__ __forceinline__ float finish(float inv, float ar, float av, float arv) {
#pragma clang fp contract(off)
  const float vbar = av * inv;
  const float corr = vbar * (ar * inv) - arv * inv;
  return vbar + corr;
}

__device__ __forceinline__ float sum8(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  return x;
}

// Load rows [row0, row0 + R) of one (b, h) into an LDS tile, zero past N.
template <bool BF16, int D, int R>
__device__ __forceinline__ void load_tile(float (*dst)[D + 1], const void* src,
                                          int64_t base, int64_t sn, int row0,
                                          int N) {
  for (int idx = threadIdx.x; idx < R * D; idx += kThreads) {
    const int r = idx / D, d = idx % D;
    const int n = row0 + r;
    dst[r][d] = n < N ? load_elem<BF16>(src, base + (int64_t)n * sn + d) : 0.0f;
  }
}

// A key (or value) tile of BN rows in registers: thread t holds the 16-byte
// pieces t, t + 256, ... of the tile (row-major, D floats per row); rows
// past N read as zero. Issued one tile ahead, so the loads of the next tile
// are in flight while the current one is computed.
template <int D, int BN>
struct TileRegs {
  static constexpr int PER = BN * D / 4 / kThreads;  // float4 per thread
  float4 x[PER];
  __device__ __forceinline__ void load(const float* base, int64_t sn, int row0, int N) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + kThreads * i;
      const int r = idx / (D / 4), c = idx % (D / 4);
      const int n = row0 + r;
      x[i] = n < N ? *reinterpret_cast<const float4*>(base + (int64_t)n * sn + 4 * c)
                   : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }
  __device__ __forceinline__ void store(float (*dst)[D + 1]) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + kThreads * i;
      const int r = idx / (D / 4), c = idx % (D / 4);
      dst[r][4 * c + 0] = x[i].x;
      dst[r][4 * c + 1] = x[i].y;
      dst[r][4 * c + 2] = x[i].z;
      dst[r][4 * c + 3] = x[i].w;
    }
  }
};

// BN keys per tile: 32 at D = 64, 16 at D = 128 (LDS below 64 KiB).
template <int D>
constexpr int key_tile() { return D == 64 ? 32 : 16; }

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void fwd_valu_kernel(FwdParams p) {
  constexpr int BN = key_tile<D>();
  constexpr int CPT = D / kTPR;  // output columns per thread
  constexpr int KPT = BN / kTPR; // keys per thread in the score phase
  static_assert(BN * D % (4 * kThreads) == 0, "tile split");
  __shared__ float sq[kBM][D + 1];
  __shared__ float sr[kBM][D + 1];
  __shared__ float sk[BN][D + 1];
  __shared__ float sv[BN][D + 1];
  __shared__ float sp[kBM][BN + 1];
  __shared__ float spr[kBM][BN + 1];

  const int i0 = blockIdx.x * kBM;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int t = threadIdx.x;
  const int i = t / kTPR;
  const int c = t % kTPR;
  const int qi = i0 + i;
  const int N = p.N;

  const float* kb = reinterpret_cast<const float*>(p.k) + b * p.k_sb + h * p.k_sh;
  const float* vb = reinterpret_cast<const float*>(p.v) + b * p.v_sb + h * p.v_sh;
  TileRegs<D, BN> kr, vr;
  kr.load(kb, p.k_sn, 0, N);
  vr.load(vb, p.v_sn, 0, N);
  load_tile<false, D, kBM>(sq, p.q, b * p.q_sb + h * p.q_sh, p.q_sn, i0, N);
  load_tile<false, D, kBM>(sr, p.rho, b * p.r_sb + h * p.r_sh, p.r_sn, i0, N);
  kr.store(sk);
  vr.store(sv);

  float m = -INFINITY, l = 0.0f, ar = 0.0f;
  float ov[CPT], orv[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) { ov[e] = 0.0f; orv[e] = 0.0f; }

  int kend = N;
  if (p.causal) kend = (i0 + kBM < N) ? i0 + kBM : N;
  const float cs = p.scale_log2;

  for (int j0 = 0; j0 < kend; j0 += BN) {
    const bool more = j0 + BN < kend;
    if (more) {   // next tile's loads in flight during this tile
      kr.load(kb, p.k_sn, j0 + BN, N);
      vr.load(vb, p.v_sn, j0 + BN, N);
    }
    __syncthreads();   // this tile (and q, rho) in LDS

    float s[KPT], r[KPT];
    bool ok[KPT];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int j = c + kTPR * u;
      float a = 0.0f, z = 0.0f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        const float kv = sk[j][d];
        a = fmaf(sq[i][d], kv, a);
        z = fmaf(sr[i][d], kv, z);
      }
      const int kj = j0 + j;
      ok[u] = qi < N && kj < N && (!p.causal || kj <= qi);
      s[u] = a * cs;
      r[u] = z;
      if (ok[u]) mx = fmaxf(mx, s[u]);
    }
    mx = max8(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = (mnew == m) ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);
    float ps = 0.0f, prs = 0.0f;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const float pj = ok[u] ? __builtin_amdgcn_exp2f(s[u] - mnew) : 0.0f;
      const float pr = pj * r[u];
      ps += pj;
      prs += pr;
      sp[i][c + kTPR * u] = pj;
      spr[i][c + kTPR * u] = pr;
    }
    ps = sum8(ps);
    prs = sum8(prs);
    l = fmaf(l, alpha, ps);
    ar = fmaf(ar, alpha, prs);
    m = mnew;
    __syncthreads();   // p and p r of the tile in LDS
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int d = c + kTPR * e;
      float a = ov[e] * alpha, z = orv[e] * alpha;
#pragma unroll 8
      for (int j = 0; j < BN; ++j) {
        const float vj = sv[j][d];
        a = fmaf(sp[i][j], vj, a);
        z = fmaf(spr[i][j], vj, z);
      }
      ov[e] = a;
      orv[e] = z;
    }
    if (more) {
      __syncthreads();   // every thread is done with this tile's K and V
      kr.store(sk);
      vr.store(sv);
    }
  }

  if (qi < N) {
    const int64_t ob = b * p.o_sb + (int64_t)qi * p.o_sn + h * p.o_sh;
    const bool any = l > 0.0f;
    const float inv = any ? 1.0f / l : 0.0f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int d = c + kTPR * e;
      const float o = any ? finish(inv, ar, ov[e], orv[e]) : 0.0f;
      if constexpr (OUT_BF16)
        reinterpret_cast<unsigned short*>(p.out)[ob + d] = f32_to_bf16_bits(o);
      else
        reinterpret_cast<float*>(p.out)[ob + d] = o;
    }
  }
}

template <int D>
hipError_t launch_valu(const FwdParams& p, bool out_bf16, hipStream_t stream) {
  const dim3 grid((p.N + kBM - 1) / kBM, p.H, p.B);
  if (out_bf16)
    hipLaunchKernelGGL((fwd_valu_kernel<D, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_valu_kernel<D, false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, int D, bool out_bf16,
                          hipStream_t stream) {
  return D == 128 ? launch_valu<128>(p, out_bf16, stream) : launch_valu<64>(p, out_bf16, stream);
}


}  // namespace parallax
