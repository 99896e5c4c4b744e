// bwd_mfma.hip -- backward of the bf16 Parallax attention prefill on the
// gfx950 matrix cores.
//
// The forward output per query i (zubnet.ai news item on Parallax, second
// paragraph) is o_i = vbar_i - C_i rho_i = vbar_i (1 + rbar_i) - u_i with
// p_ij = softmax_j(s_ij), s_ij = scale q_i.k_j, r_ij = rho_i.k_j,
// vbar = sum p v, rbar = sum p r, u = sum p r v. The pages give no backward
// pass; the chain rule on that expression, with g_i = dL/do_i,
//   a_ij = g_i.v_j,  b_i = g_i.vbar_i,  D_i = g_i.o_i + rbar_i b_i,
//   ds_ij = p_ij (a_ij (1 + rbar_i - r_ij) + b_i r_ij - D_i),
//   dr_ij = p_ij (b_i - a_ij),
// gives
//   dq_i = scale sum_j ds_ij k_j,          drho_i = sum_j dr_ij k_j,
//   dk_j = sum_i (scale ds_ij q_i + dr_ij rho_i),
//   dv_j = sum_i p_ij (1 + rbar_i - r_ij) g_i.
// A statistics pass stores per query lse2 = log2 sum_j 2^(s_ij log2 e),
// 1 + rbar_i, b_i and D_i, so both gradient kernels recompute
// p_ij = 2^(s_ij scale log2 e - lse2) exactly, with no running max. It is
// bwd_dq_kernel in statistics mode: the same S, Rk and A products, then per
// lane an online softmax over its keys summing p, p r, p a and p r a in
// fp32, since b_i = sum p a and g_i.o_i = b_i (1 + rbar_i) - sum p r a
// (6 D flops per pair; the forward would take 8 D and packed V tiles).
// From a training forward's saved o, vbar, lse2 and rbar, bwd_dq_kernel
// forms b_i and D_i itself in its prologue and publishes the statistics
// for bwd_dkv_kernel, so that path has no separate pass.
//
// bwd_dq_kernel (one workgroup per 64 queries of one (b, h), 16 per wave,
// two workgroups per CU like the forward): per 64-key tile, S^T = K Q^T,
// Rk^T = K R^T and A^T = V dO^T on bf16 MFMA (K fragments shared by the
// first two), then dS and dR elementwise, then dQ^T += K^T dS^T and
// dRho^T += K^T dR^T sharing each K^T fragment. K and V row-major tiles are
// staged by LDS-DMA, double-buffered; the K^T fragments come from the same
// K tile through the transposing LDS read.
//
// bwd_dkv_kernel (one workgroup per 16 * waves keys of one (b, h); each
// wave keeps its 16 keys' K and V rows in registers): per 32-query tile,
// S = Q K^T, R = Rho K^T (sharing the K fragments) and A = dO V^T, then
// dS, dR and P' = P o (1 + rbar - R) elementwise, then
// dK^T += Q^T (scale dS) + Rho^T dR and dV^T += dO^T P'. The row-major
// Q, rho, dO tiles and the tile's statistics are staged by LDS-DMA,
// double-buffered, from the last query tile down, so the key blocks of one
// (b, h) read each tile at about the same time; the transposed operands
// Q^T, Rho^T, dO^T (and K^T in bwd_dq_kernel) come from the same row-major
// tiles through the transposing LDS read, so nothing is packed beforehand.
//
// The two staging buffers of each kernel are separate LDS objects: the
// compiler can then tell the transposing reads of one buffer from the
// LDS-DMA into the other and does not hold them until the next tile has
// landed. Each wave waits for its own DMA before the barrier that hands the
// tile to the workgroup. The order of LDS reads and products inside a tile
// is pinned so fragments are read two products ahead of their use.
//
// Precision: the products of q.k, rho.k and dO.v are exact in fp32 (bf16
// operands); dS, dR and P' enter the second group of contractions as bf16
// (range of fp32, so loss scaling cannot overflow them), all accumulation
// fp32, gradients written fp32.
//
// Lane layouts of v_mfma_f32_16x16x32_bf16 (checked on hardware):
//   A[i][k]: lane i + 16*(k/8), element k%8
//   B[k][j]: lane j + 16*(k/8), element k%8
//   C[i][j]: lane j + 16*(i/4), register i%4
// Row-major tiles keep 16-byte chunk c of row r at slot c ^ tile_swz<D>(r);
// the contractions over D give lane group g the chunks 4 t + tile_chunk<D>(g)
// of both operands (mfma_common.h).
#include "internal.h"
#include "mfma_common.h"

namespace parallax {
namespace {

using namespace mfma;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// LDS-DMA: global -> LDS, 16 bytes per lane at dst + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned short* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

// Waits until this wave's LDS-DMA loads have written LDS; the barrier that
// follows then publishes the staged tile to the whole workgroup.
__device__ __forceinline__ void sync_staged() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Two fp32 -> two bf16 (round to nearest even), packed.
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  const f32x2_t x = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2_t));
}

// 16-byte fragment of one row of a bf16 [.., N, .., D] tensor (zero past N).
__device__ __forceinline__ bf16x8_t row_frag(const void* base, int64_t off_elems, bool valid) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const u32x4 w = valid ? *reinterpret_cast<const u32x4*>(
                              reinterpret_cast<const unsigned short*>(base) + off_elems)
                        : z;
  return __builtin_bit_cast(bf16x8_t, w);
}

// ---------------------------------------------------------------- dq, drho
// KT keys per staged tile (32 or 64): with NW = 4 the double-buffered K and
// V tiles take at most 64 KiB of LDS at D = 128, so each CU runs two
// workgroups and their per-tile barriers are independent.
template <int D, int NW, int KT, bool SAVED, bool STATS = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
  static_assert(!(SAVED && STATS), "one source of statistics");
  static_assert(KT == 32 || KT == 64, "32-key contraction steps");
  constexpr int kBM = NW * 16;     // queries per workgroup
  constexpr int NKB = KT / 16;     // 16-key blocks per tile
  constexpr int NKS = KT / 32;     // 32-key steps per tile
  constexpr int DT = D / 32;
  constexpr int DB = D / 16;
  constexpr int CPR = D / 8;
  constexpr int TILE = KT * D;
  constexpr int KPT = TILE * 2 / 1024 / NW;  // 1-KiB loads per wave per tile
  constexpr int RPK = 512 / D;               // rows per KiB
  static_assert(KPT * NW * 1024 == TILE * 2, "tile load split");

  // two buffers, each [K][V], as separate LDS objects
  __shared__ __attribute__((aligned(16))) unsigned short sm0[2 * TILE];
  __shared__ __attribute__((aligned(16))) unsigned short sm1[2 * TILE];

  const int nqb = (p.N + kBM - 1) / kBM;
  const int total = nqb * p.H * p.B;
  int lin = blockIdx.x + nqb * (blockIdx.y + p.H * blockIdx.z);
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int qbl = lin % nqb;
  const int bh = lin / nqb;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int qb = p.causal ? (nqb - 1 - qbl) : qbl;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lj = lane & 15;
  const int lg = lane >> 4;
  const int N = p.N;
  const int q0 = qb * kBM;
  const int qw0 = q0 + wave * 16;
  const int qi = qw0 + lj;
  const bool qok = qi < N;
  const float cs = p.scale_log2;

  // B operands: rows qi of Q, rho and dO (d = 32t + 8 tile_chunk(lg) .. +7)
  bf16x8_t qf[DT], rf[DT], gf[DT];
  {
    const int row = qok ? qi : 0;
    const int64_t qo = b * p.q_sb + (int64_t)row * p.q_sn + h * p.q_sh;
    const int64_t ro = b * p.r_sb + (int64_t)row * p.r_sn + h * p.r_sh;
    const int64_t go = b * p.g_sb + (int64_t)row * p.g_sn + h * p.g_sh;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int d0 = 32 * t + 8 * tile_chunk<D>(lg);
      qf[t] = row_frag(p.q, qo + d0, qok);
      rf[t] = row_frag(p.rho, ro + d0, qok);
      gf[t] = row_frag(p.dout, go + d0, qok);
    }
  }
  f32x4_t st = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (SAVED) {
    // This query's statistics from the saved forward: b = g.vbar and
    // D = g.o + rbar b over the lane's D/4 entries of g (the gf fragments),
    // then over the query's four lanes; lse2 and rbar as saved. Lane
    // group 0 publishes them for the key-block kernel.
    float gv = 0.0f, go = 0.0f;
    float2 lr = {0.0f, 0.0f};
    if (qok) {
      const float* vb = p.saved_vbar + (((int64_t)b * N + qi) * p.H + h) * D;
      const int64_t ob = b * p.so_sb + (int64_t)qi * p.so_sn + h * p.so_sh;
      lr = *reinterpret_cast<const float2*>(p.saved_lse_rbar +
                                            2 * (((int64_t)b * p.H + h) * N + qi));
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int d0 = 32 * t + 8 * tile_chunk<D>(lg);
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(vb + d0);
        const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(vb + d0 + 4);
        float o8[8];
        if (p.saved_out_bf16) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(
              reinterpret_cast<const unsigned short*>(p.saved_out) + ob + d0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o8[2 * e] = __uint_as_float(w[e] << 16);
            o8[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
          }
        } else {
          const f32x4_t o0 = *reinterpret_cast<const f32x4_t*>(
              reinterpret_cast<const float*>(p.saved_out) + ob + d0);
          const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(
              reinterpret_cast<const float*>(p.saved_out) + ob + d0 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { o8[e] = o0[e]; o8[4 + e] = o1[e]; }
        }
        const u32x4 g = __builtin_bit_cast(u32x4, gf[t]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g0 = __uint_as_float(g[e] << 16), g1 = __uint_as_float(g[e] & 0xffff0000u);
          const float vv0 = e < 2 ? v0[2 * e] : v1[2 * e - 4];
          const float vv1 = e < 2 ? v0[2 * e + 1] : v1[2 * e - 3];
          gv = fmaf(g0, vv0, fmaf(g1, vv1, gv));
          go = fmaf(g0, o8[2 * e], fmaf(g1, o8[2 * e + 1], go));
        }
      }
    }
    const int bperm32 = (lane ^ 32) << 2;
    gv += xor16(gv);
    gv += xor32(gv, bperm32);
    go += xor16(go);
    go += xor32(go, bperm32);
    st = f32x4_t{lr.x, 1.0f + lr.y, gv, go + lr.y * gv};
    if (qok && lg == 0)
      *reinterpret_cast<f32x4_t*>(p.stats_w + 4 * (((int64_t)b * p.H + h) * N + qi)) = st;
  } else if constexpr (!STATS) {
    if (qok)
      st = *reinterpret_cast<const f32x4_t*>(p.stats + 4 * (((int64_t)b * p.H + h) * N + qi));
  }
  const float lse2 = st[0], w1 = st[1], bq = st[2], dsum = st[3];   // w1 = 1 + rbar

  // staging
  const char* kbh = reinterpret_cast<const char*>(p.k) + (b * p.k_sb + h * p.k_sh) * 2;
  const char* vbh = reinterpret_cast<const char*>(p.v) + (b * p.v_sb + h * p.v_sh) * 2;
  const int64_t kspan = (int64_t)(N - 1) * p.k_sn * 2 + D * 2;
  const int64_t vspan = (int64_t)(N - 1) * p.v_sn * 2 + D * 2;
  const int64_t kstep = (int64_t)KT * p.k_sn * 2;
  const int64_t vstep = (int64_t)KT * p.v_sn * 2;
  int kdo[KPT], vdo[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int r = (KPT * wave + i) * RPK + lane / CPR;
    const int c = ((lane % CPR) ^ tile_swz<D>(r)) << 4;
    kdo[i] = r * (int)p.k_sn * 2 + c;
    vdo[i] = r * (int)p.v_sn * 2 + c;
  }
  auto stage = [&](int it, int buf) {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbh + it * kstep, kspan - it * kstep);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbh + it * vstep, vspan - it * vstep);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int blk = KPT * wave + i;
      unsigned short* const bb = buf ? sm1 : sm0;
      dma16(rk, bb + blk * 512, kdo[i]);
      dma16(rv, bb + TILE + blk * 512, vdo[i]);
    }
  };

  int kfo[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
    kfo[t] = lj * D + (((4 * t + tile_chunk<D>(lg)) ^ tile_swz<D>(lj)) << 3);
  // K^T operands straight from the row-major K tile with the transposing
  // LDS read of gfx950 (ds_read_b64_tr_b16): within each group of 16 lanes,
  // lane i receives as its element k element i % 4 of the 8 bytes addressed
  // by lane 4 k + i / 4. Lane (j, lg) addresses key row 4 lg + j / 4 at
  // head-dim entries 16 db + 4 (j % 4) .. + 3 (then the row 16 further on),
  // so lane (i, lg) receives K[4 lg + k][16 db + i] and K[16 + 4 lg + k][16 db + i],
  // k = 0..3: the A operand K^T of the 32-key contraction, in the key order
  // the dS operand has (element e <-> key 16 (e / 4) + 4 lg + e % 4).
  int tro[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int r = 4 * lg + (lj >> 2);           // key row (+ 16 for the second read)
    const int c = 2 * db + ((lj & 3) >> 1);     // 16-byte chunk of the row
    tro[db] = r * D + ((c ^ tile_swz<D>(r)) << 3) + 4 * (lj & 1);
  }
  auto tr_read = [](const unsigned short* a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(a));
  };

  f32x4_t dqa[DB], dra[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dqa[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    dra[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // Statistics mode: this lane's online softmax over its keys (base-2
  // logits x = s * scale * log2 e against the running maximum xm), with the
  // sums l = sum p, rs = sum p r, bs = sum p a, gs = sum p r a in fp32.
  float xm = -INFINITY, sl = 0.0f, srs = 0.0f, sbs = 0.0f, sgs = 0.0f;

  int kend = N;
  if (p.causal) kend = (q0 + kBM < N) ? q0 + kBM : N;
  const int ntiles = (kend + KT - 1) / KT;
  int wtiles = 0;
  if (qw0 < N) {
    const int wk = p.causal ? (qw0 + 16 < kend ? qw0 + 16 : kend) : kend;
    wtiles = (wk + KT - 1) / KT;
  }

  auto tile = [&](int j0, int buf) {
    const unsigned short* kt = buf ? sm1 : sm0;
    const unsigned short* vt = kt + TILE;
    f32x4_t s[NKB], rk[NKB], av[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      rk[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      av[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kt + 16 * kb * D + kfo[t]);
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(vt + 16 * kb * D + kfo[t]);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t], s[kb], 0, 0, 0);
        rk[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, rf[t], rk[kb], 0, 0, 0);
        av[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, gf[t], av[kb], 0, 0, 0);
      }
    }
    // pinned order: K and V fragments two products ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NKB * DT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      if (i + 2 < NKB * DT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // keys of (kb, r) for this lane: j0 + 16*kb + 4*lg + r; masked
    // probabilities are set to zero after the exponential (any scale sign)
    // key j0 + 16 kb + 4 lg + r is masked iff 16 kb + r > thr (per lane)
    const int thr = (p.causal ? min(qi, N - 1) : N - 1) - j0 - 4 * lg;
    if constexpr (STATS) {
      // masked keys take x = -inf: they neither raise the maximum nor add
      float x[NKB][4];
      float tm = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[kb][r] = 16 * kb + r > thr ? -INFINITY : s[kb][r] * cs;
          tm = fmaxf(tm, x[kb][r]);
        }
      const float mnew = fmaxf(xm, tm);
      const float alpha = (mnew == xm) ? 1.0f : __builtin_amdgcn_exp2f(xm - mnew);
      xm = mnew;
      sl *= alpha;
      srs *= alpha;
      sbs *= alpha;
      sgs *= alpha;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pe =
              x[kb][r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[kb][r] - xm);
          const float pr = pe * rk[kb][r];
          sl += pe;
          srs += pr;
          sbs = fmaf(pe, av[kb][r], sbs);
          sgs = fmaf(pr, av[kb][r], sgs);
        }
      return;
    }
    u32x4 dsw[NKS], drw[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int kb = 2 * ks + (e >> 2);
        const int r = e & 3;
        float ds[2], dr[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float pe = __builtin_amdgcn_exp2f(fmaf(s[kb][r + u], cs, -lse2));
          pe = 16 * kb + r + u > thr ? 0.0f : pe;
          const float a = av[kb][r + u], x = rk[kb][r + u];
          ds[u] = pe * fmaf(a, w1 - x, fmaf(bq, x, -dsum));
          dr[u] = pe * (bq - a);
        }
        dsw[ks][e >> 1] = pack_bf16(ds[0], ds[1]);
        drw[ks][e >> 1] = pack_bf16(dr[0], dr[1]);
      }
    // The second products run at raised wave priority: the other workgroup's
    // wave on this SIMD, in its exp / select / convert block, then issues in
    // the gaps instead of ahead of them (1-2 % on the backward).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8_t dsf = __builtin_bit_cast(bf16x8_t, dsw[ks]);
      const bf16x8_t drf = __builtin_bit_cast(bf16x8_t, drw[ks]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4_t lo = tr_read(kt + tro[db] + 32 * ks * D);
        const i16x4_t hi = tr_read(kt + tro[db] + (32 * ks + 16) * D);
        const bf16x8_t tf =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        dqa[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tf, dsf, dqa[db], 0, 0, 0);
        dra[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tf, drf, dra[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NKS * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (i + 2 < NKS * DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  stage(0, 0);
  sync_staged();
  for (int j = 0; j < ntiles; j += 2) {
    if (j + 1 < ntiles) stage(j + 1, 1);
    if (j < wtiles) tile(j * KT, 0);
    sync_staged();
    if (j + 1 >= ntiles) break;
    if (j + 2 < ntiles) stage(j + 2, 0);
    if (j + 1 < wtiles) tile((j + 1) * KT, 1);
    sync_staged();
  }

  if constexpr (STATS) {
    // Merge the four lanes of each query (keys 4 lg .. 4 lg + 3 of every
    // 16-key block), then publish {lse2, 1 + rbar, b, D} with b = g.vbar =
    // bs / l and D = g.o + rbar b = b (1 + 2 rbar) - gs / l (o = vbar (1 +
    // rbar) - sum p r v / l).
    const int bperm32 = (lane ^ 32) << 2;
    float M = fmaxf(xm, xor16(xm));
    M = fmaxf(M, xor32(M, bperm32));
    const float f = (xm == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(xm - M);
    float t4[4] = {sl * f, srs * f, sbs * f, sgs * f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t4[i] += xor16(t4[i]);
      t4[i] += xor32(t4[i], bperm32);
    }
    if (qok && lg == 0) {
      const float inv = t4[0] > 0.0f ? 1.0f / t4[0] : 0.0f;
      const float rbar = t4[1] * inv, bq = t4[2] * inv;
      const f32x4_t rec = {M + __log2f(t4[0]), 1.0f + rbar, bq,
                           fmaf(bq, fmaf(2.0f, rbar, 1.0f), -t4[3] * inv)};
      *reinterpret_cast<f32x4_t*>(p.stats_w + 4 * (((int64_t)b * p.H + h) * N + qi)) = rec;
    }
    return;
  }
  if (qok) {
    float* dq = p.dq + b * p.dq_sb + (int64_t)qi * p.dq_sn + h * p.dq_sh;
    float* dr = p.drho + b * p.dr_sb + (int64_t)qi * p.dr_sn + h * p.dr_sh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dq[16 * db + 4 * lg + r] = p.scale * dqa[db][r];
        dr[16 * db + 4 * lg + r] = dra[db][r];
      }
  }
}

// ---------------------------------------------------------------- dk, dv
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_kernel(BwdParams p) {
  constexpr int QT = 32;          // queries per tile
  constexpr int KB = 16 * NW;     // keys per workgroup
  constexpr int DT = D / 32;
  constexpr int DB = D / 16;
  constexpr int CPR = D / 8;
  constexpr int QTILE = QT * D;   // elements of one query tile
  constexpr int RPK = 512 / D;
  constexpr int KPT = QTILE * 2 / 1024 / NW;  // 1-KiB loads per wave per tile
  static_assert(KPT * NW * 1024 == QTILE * 2, "tile load split");
  // per buffer: [Q][Rho][dO] row-major tiles, statistics
  constexpr int BUF = 3 * QTILE + 512;
  __shared__ __attribute__((aligned(16))) unsigned short sm0[BUF];
  __shared__ __attribute__((aligned(16))) unsigned short sm1[BUF];

  const int nkb = (p.N + KB - 1) / KB;
  const int total = nkb * p.H * p.B;
  int lin = blockIdx.x + nkb * (blockIdx.y + p.H * blockIdx.z);
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int kbk = lin % nkb;      // causal: key block 0 sees the most queries
  const int bh = lin / nkb;
  const int h = bh % p.H;
  const int b = bh / p.H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lj = lane & 15;
  const int lg = lane >> 4;
  const int N = p.N;
  const int k0 = kbk * KB;
  const int kw0 = k0 + 16 * wave;
  const int kj = kw0 + lj;
  const bool kok = kj < N;
  const float cs = p.scale_log2;

  // B operands: rows kj of K and V (d = 32t + 8 tile_chunk(lg) .. +7)
  bf16x8_t kf[DT], vf[DT];
  {
    const int row = kok ? kj : 0;
    const int64_t ko = b * p.k_sb + (int64_t)row * p.k_sn + h * p.k_sh;
    const int64_t vo = b * p.v_sb + (int64_t)row * p.v_sn + h * p.v_sh;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int d0 = 32 * t + 8 * tile_chunk<D>(lg);
      kf[t] = row_frag(p.k, ko + d0, kok);
      vf[t] = row_frag(p.v, vo + d0, kok);
    }
  }

  // staging: wave w loads 1-KiB blocks KPT w .. KPT w + KPT - 1 of each of
  // the three tiles; lane L of block blk fills row blk * RPK + L / CPR, slot
  // L % CPR, with global chunk (L % CPR) ^ tile_swz<D>(row).
  const char* qbh = reinterpret_cast<const char*>(p.q) + (b * p.q_sb + h * p.q_sh) * 2;
  const char* rbh = reinterpret_cast<const char*>(p.rho) + (b * p.r_sb + h * p.r_sh) * 2;
  const char* gbh = reinterpret_cast<const char*>(p.dout) + (b * p.g_sb + h * p.g_sh) * 2;
  const char* sbh = reinterpret_cast<const char*>(p.stats) + ((int64_t)b * p.H + h) * N * 16;
  unsigned qdo[KPT], rdo[KPT], gdo[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int r = (KPT * wave + i) * RPK + lane / CPR;
    const unsigned c = ((lane % CPR) ^ tile_swz<D>(r)) << 4;
    qdo[i] = r * (unsigned)p.q_sn * 2 + c;
    rdo[i] = r * (unsigned)p.r_sn * 2 + c;
    gdo[i] = r * (unsigned)p.g_sn * 2 + c;
  }
  // One buffer resource per stream over the whole (b, h) slice (under 2 GiB,
  // checked by the host); a tile is selected by the 32-bit lane offset, so
  // rows past N still fall outside the resource and read as zero.
  auto span = [&](int64_t sn) { return (int64_t)(N - 1) * sn * 2 + D * 2; };
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbh, span(p.q_sn));
  const __amdgpu_buffer_rsrc_t rr_ = make_rsrc(rbh, span(p.r_sn));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gbh, span(p.g_sn));
  const __amdgpu_buffer_rsrc_t rst = make_rsrc(sbh, (int64_t)N * 16);
  // (offsets in unsigned arithmetic: one that wraps lies past the resource)
  const unsigned qstep = QT * (unsigned)p.q_sn * 2, rstep = QT * (unsigned)p.r_sn * 2;
  const unsigned gstep = QT * (unsigned)p.g_sn * 2;
  auto stage = [&](int qt, int buf) {
    unsigned short* bb = buf ? sm1 : sm0;
    const unsigned t = (unsigned)qt;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      unsigned short* d = bb + (KPT * wave + i) * 512;
      dma16(rq, d + 0 * QTILE, (int)(qdo[i] + t * qstep));
      dma16(rr_, d + 1 * QTILE, (int)(rdo[i] + t * rstep));
      dma16(rg, d + 2 * QTILE, (int)(gdo[i] + t * gstep));
    }
    if (wave == 0) dma16(rst, bb + 3 * QTILE, (int)(lane * 16u + t * (QT * 16u)));
  };

  int qfo[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
    qfo[t] = lj * D + (((4 * t + tile_chunk<D>(lg)) ^ tile_swz<D>(lj)) << 3);
  // Q^T, Rho^T and dO^T operands straight from the row-major tiles with the
  // transposing LDS read (as in bwd_dq_kernel): lane (j, lg) addresses query
  // row 4 lg + j / 4 (then the row 16 further on) at head-dim entries
  // 16 db + 4 (j % 4) .. + 3, so lane (i, lg) receives the entries
  // 16 db + i of queries 4 lg + k and 16 + 4 lg + k, k = 0..3: the A operand
  // of the 32-query contraction in the query order of the dS, dR and P'
  // operands (element e <-> query 16 (e / 4) + 4 lg + e % 4).
  int tro[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int r = 4 * lg + (lj >> 2);
    const int c = 2 * db + ((lj & 3) >> 1);
    tro[db] = r * D + ((c ^ tile_swz<D>(r)) << 3) + 4 * (lj & 1);
  }
  auto tr_read = [](const unsigned short* a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(a));
  };
  auto tr_frag = [&](const unsigned short* tile, int db) {
    const i16x4_t lo = tr_read(tile + tro[db]);
    const i16x4_t hi = tr_read(tile + tro[db] + 16 * D);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x4_t dka[DB], dva[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dka[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    dva[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int nqt = (N + QT - 1) / QT;
  const int qt0 = p.causal ? k0 / QT : 0;

  auto tile = [&](int qt, int buf) {
    const unsigned short* bb = buf ? sm1 : sm0;
    const int q0 = qt * QT;
    f32x4_t s[2], rr[2], av[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      rr[qb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      av[qb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int o = 16 * qb * D + qfo[t];
        const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(bb + 0 * QTILE + o);
        const bf16x8_t ra = *reinterpret_cast<const bf16x8_t*>(bb + 1 * QTILE + o);
        const bf16x8_t ga = *reinterpret_cast<const bf16x8_t*>(bb + 2 * QTILE + o);
        s[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[t], s[qb], 0, 0, 0);
        rr[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra, kf[t], rr[qb], 0, 0, 0);
        av[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga, vf[t], av[qb], 0, 0, 0);
      }
    }
    // statistics of the eight queries this lane meets
    f32x4_t stv[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        stv[qb][r] = *reinterpret_cast<const f32x4_t*>(bb + 3 * QTILE + 8 * (16 * qb + 4 * lg + r));
    // pinned order: fragments two products ahead, one statistics read per step
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      if (i + 2 < 2 * DT) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // lane (key lj, group lg) holds queries q0 + 16*qb + 4*lg + r
    // causal: query q0 + c is masked for this lane's key iff c < thr; rows
    // past N need no mask (their q, rho, dO and statistics read as zero,
    // which makes dS = dR = P' = 0)
    const int thr = p.causal ? kj - q0 : -1;
    unsigned dsh[4], drh[4], pvh[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        float ds[2], dr[2], pv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int ql = 16 * qb + 4 * lg + r + u;
          const f32x4_t& st = stv[qb][r + u];
          float pe = __builtin_amdgcn_exp2f(fmaf(s[qb][r + u], cs, -st[0]));
          pe = ql < thr ? 0.0f : pe;
          const float a = av[qb][r + u], x = rr[qb][r + u];
          const float w = st[1] - x;                       // st[1] = 1 + rbar
          ds[u] = p.scale * pe * fmaf(a, w, fmaf(st[2], x, -st[3]));
          dr[u] = pe * (st[2] - a);
          pv[u] = pe * w;
        }
        dsh[2 * qb + (r >> 1)] = pack_bf16(ds[0], ds[1]);
        drh[2 * qb + (r >> 1)] = pack_bf16(dr[0], dr[1]);
        pvh[2 * qb + (r >> 1)] = pack_bf16(pv[0], pv[1]);
      }
    // element e of the 32-query contraction <-> query 16*(e/4) + 4*lg + e%4
    const bf16x8_t dsf = __builtin_bit_cast(bf16x8_t, u32x4{dsh[0], dsh[1], dsh[2], dsh[3]});
    const bf16x8_t drf = __builtin_bit_cast(bf16x8_t, u32x4{drh[0], drh[1], drh[2], drh[3]});
    const bf16x8_t pvf = __builtin_bit_cast(bf16x8_t, u32x4{pvh[0], pvh[1], pvh[2], pvh[3]});
    __builtin_amdgcn_s_setprio(1);   // as in bwd_dq_kernel
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8_t qt_ = tr_frag(bb + 0 * QTILE, db);
      const bf16x8_t rt_ = tr_frag(bb + 1 * QTILE, db);
      const bf16x8_t gt_ = tr_frag(bb + 2 * QTILE, db);
      dka[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt_, dsf, dka[db], 0, 0, 0);
      dka[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rt_, drf, dka[db], 0, 0, 0);
      dva[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gt_, pvf, dva[db], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      if (db + 2 < DB) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Query tiles are walked from the last one down to the first this block
  // sees, so all key blocks of one (b, h) -- which run together on one XCD
  // -- read the same query tile at about the same time and share it in L2
  // (walking upwards from each block's own diagonal would spread them over
  // the whole q / rho / dO stream of the head).
  if (qt0 < nqt) {
    stage(nqt - 1, 0);
    sync_staged();
    for (int qt = nqt - 1; qt >= qt0; qt -= 2) {
      if (qt - 1 >= qt0) stage(qt - 1, 1);
      tile(qt, 0);
      sync_staged();
      if (qt - 1 < qt0) break;
      if (qt - 2 >= qt0) stage(qt - 2, 0);
      tile(qt - 1, 1);
      sync_staged();
    }
  }

  if (kok) {
    float* dk = p.dk + b * p.dk_sb + (int64_t)kj * p.dk_sn + h * p.dk_sh;
    float* dv = p.dv + b * p.dv_sb + (int64_t)kj * p.dv_sn + h * p.dv_sh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dk[16 * db + 4 * lg + r] = dka[db][r];
        dv[16 * db + 4 * lg + r] = dva[db][r];
      }
  }
}

// dq, drho: 4 waves per workgroup, 64-key tiles (1 % faster than 32-key
// ones). dk, dv: NW waves (4: 64 keys per workgroup and 50 KiB of LDS, so
// each CU runs two workgroups whose barriers are independent; one 8-wave
// workgroup per CU measured 7 % slower over the whole backward).
constexpr int kDqWaves = 4;
constexpr int kDqKeys = 64;

template <int D, int NW>
hipError_t launch(const BwdParams& p, hipStream_t stream) {
  const dim3 gq((p.N + kDqWaves * 16 - 1) / (kDqWaves * 16), p.H, p.B);
  if (p.saved_out != nullptr)
    hipLaunchKernelGGL((bwd_dq_kernel<D, kDqWaves, kDqKeys, true>), gq, dim3(64 * kDqWaves), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, kDqWaves, kDqKeys, false>), gq, dim3(64 * kDqWaves),
                       0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gk((p.N + NW * 16 - 1) / (NW * 16), p.H, p.B);
  hipLaunchKernelGGL((bwd_dkv_kernel<D, NW>), gk, dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_stats(const BwdParams& p, hipStream_t stream) {
  const dim3 gq((p.N + kDqWaves * 16 - 1) / (kDqWaves * 16), p.H, p.B);
  hipLaunchKernelGGL((bwd_dq_kernel<D, kDqWaves, kDqKeys, false, true>), gq,
                     dim3(64 * kDqWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, int D, hipStream_t stream) {
  return D == 128 ? launch<128, 4>(p, stream) : launch<64, 4>(p, stream);
}

hipError_t launch_bwd_stats_bf16(const BwdParams& p, int D, hipStream_t stream) {
  return D == 128 ? launch_stats<128>(p, stream) : launch_stats<64>(p, stream);
}

}  // namespace parallax
