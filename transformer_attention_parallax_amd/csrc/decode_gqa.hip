// decode_gqa.hip -- Parallax attention decode with grouped query heads and
// an optional paged KV cache (bf16 inputs, gfx950).
//
// Same computation as decode.hip (one streaming pass over K and V feeds
// both the softmax branch and the covariance branch; zubnet.ai news item on
// Parallax, second paragraph), generalised in two ways:
//  * G = Hq / Hkv query heads (each with its own probe rho) share one
//    key-value head. One workgroup streams the keys of one (b, kv head,
//    split) once and keeps G online-softmax states: every K row feeds 2G dot
//    products (q_g.k and rho_g.k), every V row 2G accumulations. Bytes per
//    token are those of one kv head, so the arithmetic per byte grows by G.
//  * Paged cache: position l of sequence b lives in page
//    block_table[b][l / P] at row l % P; element (page, t, hk, d) at
//    page*kv_sb + t*kv_sl + hk*kv_sh + d. With P a multiple of 8 the rows a
//    wave loads in one unrolled slot share one page, so the page index is a
//    scalar (wave-uniform) load. Keys whose page index falls outside
//    [0, num_pages) are skipped, never read.
// Without a block table the cache is contiguous, element (b, hk, l, d) at
// b*kv_sb + hk*kv_sh + l*kv_sl + d.
//
// Lane layout and state as in decode.hip: LPK = D/8 lanes hold one key row
// (one 16-byte load each), KPW = 64/LPK rows per wave-wide load, U unrolled
// slots per lane; per lane group and query head fp32 (m, l, A_r) in base-2
// logit units and this lane's D/LPK entries of A_v and A_rv. Split records
// [m, l, A_r, 0, A_v, A_rv] per (b, query head, split) are merged by the
// combine kernel of decode.hip.
#include "decode_common.h"

namespace parallax {
namespace {

using namespace dec;

template <int D, int G, bool PAGED, bool SPLIT, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void decode_gqa_kernel(DecodeParams p) {
  constexpr int EPL = 8;
  constexpr int LPK = D / EPL;        // lanes per key row
  constexpr int KPW = 64 / LPK;       // key rows per wave-wide load
  constexpr int NG = kWaves * KPW;    // lane groups per workgroup
  constexpr int U = G == 1 ? 8 : (G <= 4 ? 4 : 2);
  constexpr int STEP = kWaves * U * KPW;

  __shared__ float sm_m[NG], sm_l[NG], sm_ar[NG];
  __shared__ float sm_v[NG][D];
  __shared__ float sm_rv[NG][D];

  const int split = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int grp = lane / LPK;
  const int d0 = (lane % LPK) * EPL;

  int len = p.Lmax;
  if (p.seqlens != nullptr) {
    const int sl = p.seqlens[b];
    len = sl < len ? sl : len;
  }
  if (len < 0) len = 0;
  const int j0 = split * p.chunk;
  int j1 = j0 + p.chunk;
  if (j1 > len) j1 = len;

  u32x4 qw[G], rw[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int hq = hk * G + g;
    qw[g] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned short*>(p.q) +
                                            b * p.q_sb + hq * p.q_sh + d0);
    rw[g] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned short*>(p.rho) +
                                            b * p.r_sb + hq * p.r_sh + d0);
  }
  const float c = p.scale_log2;
  const unsigned short* kbase = reinterpret_cast<const unsigned short*>(p.k);
  const unsigned short* vbase = reinterpret_cast<const unsigned short*>(p.v);
  const int64_t head_off = PAGED ? hk * p.kv_sh + d0 : b * p.kv_sb + hk * p.kv_sh + d0;
  const int32_t* bt = PAGED ? p.block_table + b * p.bt_sb : nullptr;

  float m[G], l[G], ar[G], av[G][EPL], arv[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
    ar[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) { av[g][e] = 0.0f; arv[g][e] = 0.0f; }
  }

  const int nsteps = j1 > j0 ? (j1 - j0 + STEP - 1) / STEP : 0;
  for (int t = 0; t < nsteps; ++t) {
    // first row of slot u for this wave (wave-uniform): kb + u*KPW
    const int kb = j0 + t * STEP + wave * (U * KPW);
    u32x4 kw[U], vw[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row0 = kb + u * KPW;
      const int key = row0 + grp;
      int64_t roff = 0;
      bool valid = row0 < j1;
      if constexpr (PAGED) {
        int pg = -1;
        if (valid) pg = bt[row0 / p.page];      // scalar load, uniform index
        valid = valid && pg >= 0 && pg < p.num_pages;
        roff = (int64_t)pg * p.kv_sb + (int64_t)(key % p.page) * p.kv_sl;
      } else {
        roff = (int64_t)key * p.kv_sl;
      }
      ok[u] = valid && key < j1;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kw[u] = ok[u] ? load16(kbase + head_off + roff) : z;
      vw[u] = ok[u] ? load16(vbase + head_off + roff) : z;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[U], r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u] = group_sum<LPK>(dot_bf16(qw[g], kw[u])) * c;
        r[u] = group_sum<LPK>(dot_bf16(rw[g], kw[u]));
      }
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = ok[u] ? fmaxf(mx, s[u]) : mx;
      const float alpha = (mx == m[g]) ? 1.0f : __builtin_amdgcn_exp2f(m[g] - mx);
      m[g] = mx;
      l[g] *= alpha;
      ar[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) { av[g][e] *= alpha; arv[g][e] *= alpha; }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pj = ok[u] ? __builtin_amdgcn_exp2f(s[u] - m[g]) : 0.0f;
        const float pr = pj * r[u];
        l[g] += pj;
        ar[g] += pr;
        float x[EPL];
        unpack_bf16(vw[u], x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          av[g][e] = fmaf(pj, x[e], av[g][e]);
          arv[g][e] = fmaf(pr, x[e], arv[g][e]);
        }
      }
    }
  }

  // Merge the NG lane-group states of each query head in turn.
  const int gid = wave * KPW + grp;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if ((lane % LPK) == 0) {
      sm_m[gid] = m[g];
      sm_l[gid] = l[g];
      sm_ar[gid] = ar[g];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      sm_v[gid][d0 + e] = av[g][e];
      sm_rv[gid][d0 + e] = arv[g][e];
    }
    __syncthreads();
    if (tid < D) {
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < NG; ++q) M = fmaxf(M, sm_m[q]);
      float L = 0.0f, AR = 0.0f, AV = 0.0f, ARV = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const float mq = sm_m[q];
          const float w = (mq == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mq - M);
          L = fmaf(w, sm_l[q], L);
          AR = fmaf(w, sm_ar[q], AR);
          AV = fmaf(w, sm_v[q][tid], AV);
          ARV = fmaf(w, sm_rv[q][tid], ARV);
        }
      }
      const int hq = hk * G + g;
      if constexpr (SPLIT) {
        constexpr int REC = decode_record_floats(D);
        float* rec = p.ws + ((int64_t)(b * p.H + hq) * p.nsplit + split) * REC;
        if (tid == 0) {
          rec[0] = M;
          rec[1] = L;
          rec[2] = AR;
          rec[3] = 0.0f;
        }
        rec[4 + tid] = AV;
        rec[4 + D + tid] = ARV;
      } else {
        store_out<OUT_BF16>(p.out, b * p.o_sb + hq * p.o_sh + tid, finish(L, AR, AV, ARV));
      }
    }
    __syncthreads();
  }
}

template <int D, int G, bool PAGED>
hipError_t launch_g(const DecodeParams& p, bool out_bf16, hipStream_t stream) {
  const dim3 grid(p.nsplit, p.Hkv, p.B);
  if (p.nsplit > 1) {
    hipLaunchKernelGGL((decode_gqa_kernel<D, G, PAGED, true, false>), grid, dim3(kThreads), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_combine(p, D, out_bf16, stream);
  }
  if (out_bf16)
    hipLaunchKernelGGL((decode_gqa_kernel<D, G, PAGED, false, true>), grid, dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((decode_gqa_kernel<D, G, PAGED, false, false>), grid, dim3(kThreads), 0,
                       stream, p);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_d(const DecodeParams& p, int group, bool out_bf16, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<D, 1, PAGED>(p, out_bf16, stream);
    case 2: return launch_g<D, 2, PAGED>(p, out_bf16, stream);
    case 4: return launch_g<D, 4, PAGED>(p, out_bf16, stream);
    default: return launch_g<D, 8, PAGED>(p, out_bf16, stream);
  }
}

}  // namespace

hipError_t launch_decode_gqa(const DecodeParams& p, int D, int group, bool out_bf16,
                             hipStream_t stream) {
  const bool paged = p.block_table != nullptr;
  if (D == 128)
    return paged ? launch_d<128, true>(p, group, out_bf16, stream)
                 : launch_d<128, false>(p, group, out_bf16, stream);
  return paged ? launch_d<64, true>(p, group, out_bf16, stream)
               : launch_d<64, false>(p, group, out_bf16, stream);
}

}  // namespace parallax
