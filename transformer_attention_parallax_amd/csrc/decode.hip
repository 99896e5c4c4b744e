// decode.hip -- Parallax attention decode on gfx950 (one query per sequence).
//
// Both branches of Parallax attention (softmax attention, and the
// key-value covariance contracted with the probe rho) are accumulated in one
// streaming pass over the KV cache: the zubnet.ai news item on Parallax
// (second paragraph) states that the two branches reuse the same KV stream,
// and the encorp.ai blog ("Integraciones de IA personalizadas tras la
// atencion Parallax", section on Hopper GPUs) adds that the extra arithmetic
// rides on the memory traffic softmax attention already pays for.
//
// Per (b, h) the kernel keeps, in fp32 and in base-2 logit units,
//   m    running max of s_j = scale*log2(e) * q.k_j
//   l    sum 2^(s_j - m)
//   A_r  sum 2^(s_j - m) r_j,          r_j = rho . k_j
//   A_v  sum 2^(s_j - m) v_j           (D values)
//   A_rv sum 2^(s_j - m) r_j v_j       (D values)
// and finishes o = vbar (1 + rbar) - A_rv / l with vbar = A_v / l,
// rbar = A_r / l, which equals vbar - C rho (C the softmax-weighted
// value-key covariance) because the weights sum to one.
//
// Work decomposition (HBM-bound: 4*D bytes of bf16 K+V per key, 8*D flops):
//  * grid (splits, H, B); one 256-thread workgroup streams one contiguous
//    key range of one (b, h).
//  * A key row (D elements, 16*LPK bytes) is read by LPK lanes with one
//    16-byte load each, so one wave-wide load instruction reads KPW = 64/LPK
//    consecutive rows (1 KiB, fully coalesced). The same registers feed both
//    dot products q.k and rho.k; the same V registers feed both A_v and
//    A_rv. Nothing is staged through LDS: the load layout already is the
//    compute layout, so LDS would only add traffic.
//  * Each group of LPK lanes owns one key per unrolled slot and its own
//    online-softmax state; the dot products are reduced inside the group
//    with DPP row permutes (every lane ends with identical bits). Groups,
//    then waves, are merged through LDS at the end with the same
//    rescale-and-add rule the split combine uses.
//  * Each lane issues U independent 16-byte K loads and U V loads per step
//    before consuming any, which keeps enough bytes in flight per CU.
//  * fp32 prefill reuses the kernel (rows mode, fp32 instantiations only):
//    stream z is query row z % N of sequence z / N and sees the keys of its
//    sequence up to the row (causal) or all N; one workgroup per (row, head).
#include "decode_common.h"

namespace parallax {
namespace {

using namespace dec;

constexpr int kUnroll = 8;
// Unsplit bf16 streams of at least kCapMinKeys keys run one workgroup per
// CU: kCapLdsBytes of dynamic LDS plus the kernel's own (about 17 KiB) is
// more than half of a CU's 160 KiB.
constexpr int kCapMinKeys = 4096;
constexpr size_t kCapLdsBytes = 96 * 1024;

// Input element traits: EPL elements per 16-byte load.
template <bool BF16> struct InT;
template <> struct InT<true> {
  static constexpr int EPL = 8;
  static constexpr int kBytes = 2;
  __device__ static float dot(const u32x4& a, const u32x4& b) { return dot_bf16(a, b); }
  __device__ static void unpack(const u32x4& w, float* x) { unpack_bf16(w, x); }
};
template <> struct InT<false> {
  static constexpr int EPL = 4;
  static constexpr int kBytes = 4;
  __device__ static float dot(const u32x4& a, const u32x4& b) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), s);
    return s;
  }
  __device__ static void unpack(const u32x4& w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
};

// CORR = false: plain softmax attention (rho == NULL): no rho.k products and
// no A_r, A_rv sums; the records and the output are those of rho = 0.
template <bool BF16, int D, bool SPLIT, bool OUT_BF16, bool CORR = true, int UNROLL = kUnroll>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  using In = InT<BF16>;
  constexpr int EPL = In::EPL;
  constexpr int LPK = D / EPL;         // lanes per key row
  constexpr int KPW = 64 / LPK;        // key rows per wave-wide load
  constexpr int NG = kWaves * KPW;     // online-softmax groups per workgroup
  constexpr int U = UNROLL;
  constexpr int STEP = kWaves * U * KPW;  // keys per workgroup step
  static_assert(LPK >= 4 && LPK <= 32, "unsupported row split");

  __shared__ float sm_m[NG], sm_l[NG], sm_ar[NG];
  __shared__ float sm_v[NG][D];
  __shared__ float sm_rv[NG][D];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int grp = lane / LPK;
  const int d0 = (lane % LPK) * EPL;

  // Query rows as streams (the fp32 prefill): stream b is row `row` of
  // sequence `sb`, whose keys are the sequence's (causal: up to the row).
  int sb = b, row = 0;
  int len = p.Lmax;
  if constexpr (!BF16) {
    if (p.rows > 0) {
      sb = b / p.rows;
      row = b - sb * p.rows;
      if (p.causal_rows && row + 1 < len) len = row + 1;
    }
  }
  if (p.seqlens != nullptr) {
    const int sl = p.seqlens[b];
    len = sl < len ? sl : len;
  }
  if (len < 0) len = 0;
  const int j0 = split * p.chunk;
  int j1 = j0 + p.chunk;
  if (j1 > len) j1 = len;

  const char* qp = reinterpret_cast<const char*>(p.q) +
                   (sb * p.q_sb + row * p.q_sn + h * p.q_sh + d0) * In::kBytes;
  const char* rp = CORR ? reinterpret_cast<const char*>(p.rho) +
                              (sb * p.r_sb + row * p.r_sn + h * p.r_sh + d0) * In::kBytes
                       : qp;
  const int64_t kv_off = (sb * p.kv_sb + h * p.kv_sh + d0) * In::kBytes;
  const char* kp = reinterpret_cast<const char*>(p.k) + kv_off;
  const char* vp = reinterpret_cast<const char*>(p.v) + kv_off;
  const int64_t row_bytes = p.kv_sl * In::kBytes;

  const u32x4 qw = *reinterpret_cast<const u32x4*>(qp);
  const u32x4 rw = CORR ? *reinterpret_cast<const u32x4*>(rp) : u32x4{0u, 0u, 0u, 0u};
  const float c = p.scale_log2;

  float m = -INFINITY, l = 0.0f, ar = 0.0f;
  float av[EPL], arv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) { av[e] = 0.0f; arv[e] = 0.0f; }

  // first key of this lane's group in the current step, slot u adds u*KPW
  int key = j0 + wave * (U * KPW) + grp;
  const int nfull = j1 > j0 ? (j1 - j0) / STEP : 0;

  for (int t = 0; t < nfull; ++t, key += STEP) {
    u32x4 kw[U], vw[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      kw[u] = load16(kp + (int64_t)(key + u * KPW) * row_bytes);
#pragma unroll
    for (int u = 0; u < U; ++u)
      vw[u] = load16(vp + (int64_t)(key + u * KPW) * row_bytes);
    float s[U], r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[u] = In::dot(qw, kw[u]);
      r[u] = CORR ? In::dot(rw, kw[u]) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[u] = group_sum<LPK>(s[u]) * c;
      if constexpr (CORR) r[u] = group_sum<LPK>(r[u]);
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u]);
    const float alpha = __builtin_amdgcn_exp2f(m - mx);  // 0 on the first step
    m = mx;
    l *= alpha;
    ar *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      av[e] *= alpha;
      if constexpr (CORR) arv[e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pj = __builtin_amdgcn_exp2f(s[u] - m);
      const float pr = pj * r[u];
      l += pj;
      ar += pr;
      float x[EPL];
      In::unpack(vw[u], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        av[e] = fmaf(pj, x[e], av[e]);
        if constexpr (CORR) arv[e] = fmaf(pr, x[e], arv[e]);
      }
    }
  }

  if (key < j1) {
    // Last, partial step: rows at or past j1 are neither loaded nor counted.
    // Validity is uniform over the LPK lanes of a group (same key), so the
    // group reductions below never mix valid and invalid rows.
    u32x4 kw[U], vw[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ok[u] = (key + u * KPW) < j1;
      const u32x4 z = {0u, 0u, 0u, 0u};
      kw[u] = ok[u] ? load16(kp + (int64_t)(key + u * KPW) * row_bytes) : z;
      vw[u] = ok[u] ? load16(vp + (int64_t)(key + u * KPW) * row_bytes) : z;
    }
    float s[U], r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[u] = group_sum<LPK>(In::dot(qw, kw[u])) * c;
      r[u] = CORR ? group_sum<LPK>(In::dot(rw, kw[u])) : 0.0f;
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = ok[u] ? fmaxf(mx, s[u]) : mx;
    const float alpha = (mx == m) ? 1.0f : __builtin_amdgcn_exp2f(m - mx);
    m = mx;
    l *= alpha;
    ar *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      av[e] *= alpha;
      if constexpr (CORR) arv[e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pj = ok[u] ? __builtin_amdgcn_exp2f(s[u] - m) : 0.0f;
      const float pr = pj * r[u];
      l += pj;
      ar += pr;
      float x[EPL];
      In::unpack(vw[u], x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        av[e] = fmaf(pj, x[e], av[e]);
        if constexpr (CORR) arv[e] = fmaf(pr, x[e], arv[e]);
      }
    }
  }

  // Merge the NG group states of this workgroup.
  const int gid = wave * KPW + grp;
  if ((lane % LPK) == 0) {
    sm_m[gid] = m;
    sm_l[gid] = l;
    sm_ar[gid] = ar;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    sm_v[gid][d0 + e] = av[e];
    sm_rv[gid][d0 + e] = arv[e];
  }
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < NG; ++g) M = fmaxf(M, sm_m[g]);
    float L = 0.0f, AR = 0.0f, AV = 0.0f, ARV = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float mg = sm_m[g];
        const float w = (mg == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mg - M);
        L = fmaf(w, sm_l[g], L);
        AR = fmaf(w, sm_ar[g], AR);
        AV = fmaf(w, sm_v[g][tid], AV);
        ARV = fmaf(w, sm_rv[g][tid], ARV);
      }
    }
    if constexpr (SPLIT) {
      constexpr int REC = decode_record_floats(D);
      float* rec = p.ws + ((int64_t)(b * p.H + h) * p.nsplit + split) * REC;
      if (tid == 0) {
        rec[0] = M;
        rec[1] = L;
        rec[2] = AR;
        rec[3] = 0.0f;
      }
      rec[4 + tid] = AV;
      rec[4 + D + tid] = ARV;
    } else {
      store_out<OUT_BF16>(p.out, sb * p.o_sb + row * p.o_sn + h * p.o_sh + tid,
                          finish(L, AR, AV, ARV));
    }
  }
}

// Max (MAX) or sum over the D threads of a block; every thread gets the
// result. part holds one partial per wave and is free again on return.
template <int D, bool MAX>
__device__ __forceinline__ float block_reduce(float x, float* part) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = MAX ? fmaxf(x, y) : x + y;
  }
  if constexpr (D > 64) {
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    x = part[0];
#pragma unroll
    for (int i = 1; i < D / 64; ++i) x = MAX ? fmaxf(x, part[i]) : x + part[i];
    __syncthreads();
  }
  return x;
}

// Merge the split records of one (b, h): rescale each by 2^(m_s - M) and add.
// Every load the merge needs for up to kPreSplits splits is issued at the
// start: thread d reads the scalars (m, l, A_r) of split d once and its
// head-dim entry of the value sums of splits 0 .. kPreSplits - 1, so the
// merge waits on about one memory latency (the records were just written and
// sit in L2). Splits beyond (a long context split finely) are read after the
// weights are known, with independent loads per split. Sums run in split
// order, as they would with all loads in one loop.
constexpr int kPreSplits = 16;
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(D) void combine_kernel(DecodeParams p) {
  constexpr int REC = decode_record_floats(D);
  __shared__ float wts[kMaxDecodeSplits];
  __shared__ float part[D / 64];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int ns = p.nsplit;
  const float* rec = p.ws + (int64_t)(b * p.H + h) * ns * REC;
  float av[kPreSplits], arv[kPreSplits];
#pragma unroll
  for (int s = 0; s < kPreSplits; ++s) {
    av[s] = 0.0f;
    arv[s] = 0.0f;
    if (s < ns) {
      av[s] = rec[(int64_t)s * REC + 4 + d];
      arv[s] = rec[(int64_t)s * REC + 4 + D + d];
    }
  }
  float m0 = -INFINITY, l0 = 0.0f, r0 = 0.0f;   // scalars of split d
  if (d < ns) {
    const float* r = rec + (int64_t)d * REC;
    m0 = r[0];
    l0 = r[1];
    r0 = r[2];
  }
  float M = m0;
  for (int s = d + D; s < ns; s += D) M = fmaxf(M, rec[(int64_t)s * REC]);
  M = block_reduce<D, true>(M, part);
  float L = 0.0f, AR = 0.0f;
  if (d < ns) {
    const float w = (m0 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m0 - M);
    wts[d] = w;
    L = fmaf(w, l0, L);
    AR = fmaf(w, r0, AR);
  }
  for (int s = d + D; s < ns; s += D) {
    const float* r = rec + (int64_t)s * REC;
    const float ms = r[0];
    const float w = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
    wts[s] = w;
    L = fmaf(w, r[1], L);
    AR = fmaf(w, r[2], AR);
  }
  L = block_reduce<D, false>(L, part);
  AR = block_reduce<D, false>(AR, part);
  __syncthreads();
  float AV = 0.0f, ARV = 0.0f;
#pragma unroll
  for (int s = 0; s < kPreSplits; ++s) {
    if (s < ns) {
      const float w = wts[s];
      AV = fmaf(w, av[s], AV);
      ARV = fmaf(w, arv[s], ARV);
    }
  }
#pragma unroll 8
  for (int s = kPreSplits; s < ns; ++s) {
    const float w = wts[s];
    const float* r = rec + (int64_t)s * REC;
    AV = fmaf(w, r[4 + d], AV);
    ARV = fmaf(w, r[4 + D + d], ARV);
  }
  store_out<OUT_BF16>(p.out, b * p.o_sb + h * p.o_sh + d,
                      finish(L, AR, AV, ARV));
}

template <bool BF16, int D, bool CORR>
hipError_t launch_typed(const DecodeParams& p, bool out_bf16,
                        hipStream_t stream) {
  const dim3 grid(p.nsplit, p.H, p.B);
  if (p.nsplit > 1) {
    // Short bf16 key ranges (the few-stream case) issue 16 loads of K and
    // 16 of V per lane per step instead of 8, so a 256-key range is one
    // round trip to memory. Measured at batch 1 with 16 heads, D 128: 2048,
    // 4096 and 8192 keys in 256- and 512-key ranges 4-7 % faster; ranges of
    // 1024 keys and more 2-5 % slower, so they keep 8.
    bool deep = false;
    if constexpr (BF16) deep = p.chunk <= 512;
    if (deep)
      hipLaunchKernelGGL((decode_kernel<BF16, D, true, false, CORR, BF16 ? 2 * kUnroll : kUnroll>),
                         grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_kernel<BF16, D, true, false, CORR>), grid,
                         dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_combine(p, D, out_bf16, stream);
  }
  // One workgroup per CU for long bf16 streams: the reserved (unused)
  // dynamic LDS keeps a second workgroup off the CU. Measured with 256 / 64
  // sequences x 16 heads: 8192 and 32768 keys 1-2 % faster than four per CU;
  // at 2048 keys no gain, at 512 and 128 keys 10 and 49 % slower (short
  // streams need many workgroups in flight to hide their start-up).
  size_t lds = 0;
  if constexpr (BF16) lds = p.Lmax >= kCapMinKeys ? kCapLdsBytes : 0;
  if (out_bf16)
    hipLaunchKernelGGL((decode_kernel<BF16, D, false, true, CORR>), grid,
                       dim3(kThreads), lds, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<BF16, D, false, false, CORR>), grid,
                       dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_corr(const DecodeParams& p, bool out_bf16, hipStream_t stream) {
  return p.rho != nullptr ? launch_typed<BF16, D, true>(p, out_bf16, stream)
                          : launch_typed<BF16, D, false>(p, out_bf16, stream);
}

}  // namespace

hipError_t launch_decode_combine(const DecodeParams& p, int D, bool out_bf16,
                                 hipStream_t stream) {
  const dim3 cgrid(p.H, p.B);
  if (D == 128) {
    if (out_bf16)
      hipLaunchKernelGGL((combine_kernel<128, true>), cgrid, dim3(128), 0, stream, p);
    else
      hipLaunchKernelGGL((combine_kernel<128, false>), cgrid, dim3(128), 0, stream, p);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((combine_kernel<64, true>), cgrid, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL((combine_kernel<64, false>), cgrid, dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int D, bool in_bf16,
                         bool out_bf16, hipStream_t stream) {
  if (D == 128)
    return in_bf16 ? launch_corr<true, 128>(p, out_bf16, stream)
                   : launch_corr<false, 128>(p, out_bf16, stream);
  return in_bf16 ? launch_corr<true, 64>(p, out_bf16, stream)
                 : launch_corr<false, 64>(p, out_bf16, stream);
}

}  // namespace parallax
