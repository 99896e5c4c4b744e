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
// Four contractions per (query block, key tile), all on MFMA
// (v_mfma_f32_16x16x32_{bf16,f16}) with fp32 accumulation:
//   S^T  = K Q^T    and  Rk^T = K R^T        bf16 (products exact in fp32)
//   O_v^T  += V^T P^T  and  O_rv^T += V^T (P o Rk)^T     fp16
// The transposed forms put one query per lane column, so the per-query
// softmax state is a per-lane scalar and row reductions exchange values
// between the four lanes that share a query. Each K fragment read from LDS
// feeds both S^T and Rk^T; each V^T fragment feeds both O_v^T and O_rv^T,
// so the two branches share one pass over K and V on the matrix cores.
//
// Precision. p and p*r enter the second pair of contractions as fp16
// (11-bit significand), V converted from bf16 to fp16 once, by a packing
// kernel that runs first (exact for |v| in [2^-14, 65504]). l and R are summed from the same fp16-rounded
// values the matrix cores consume, so vbar and the covariance term use the
// same weights and the cancellation in vbar * rbar - O_rv / l stays benign.
// (bf16 probabilities miss the 2e-2 budget on the large-probe 1.7B-model
// workload.) r enters shifted by a per-query constant c, its softmax-
// weighted mean over the first key tile: the covariance, hence the output,
// does not depend on c, and |p (r - c)| then follows the spread of r rather
// than its size. Exponents are taken against a reference max m_ref + 8 that is
// only raised when a row's max exceeds it, so p <= 1 always, |p r| <= |r|,
// and the accumulators are rescaled only when some row's max grows by more
// than 2^8; the scale cancels in every ratio of the output formula.
//
// Tiling. 16 query rows per wave, 4 waves (64 rows) per workgroup, one
// wave per SIMD; <= 256 registers per lane and 64 KiB of LDS, so each CU
// runs two workgroups and each SIMD one wave of each. The two workgroups
// pass their per-tile barriers independently, so one wave's exp / convert
// work overlaps the other's matrix work (one 8-wave workgroup per CU, with
// both waves of a SIMD held in step by its barriers, measured 4-7 % slower).
// Key tiles of 64 keys are double-buffered in LDS:
//   K   [64][D] bf16, 16-byte chunk c of row j stored at chunk c ^ (j % (D/8));
//   V^T [D][64] fp16, keys reordered inside each 32-key group so that the
//       eight keys one lane feeds to a P V contraction are contiguous (one
//       16-byte load per fragment), 16-byte unit u of row d stored at
//       unit u ^ ((d >> 1) & 7);
// The gfx950 LDS serves a 16-byte-per-lane load 16 lanes at a time from 64
// banks, so the 16 lanes of a fragment load must touch 16 distinct 16-byte
// bank groups of a 256-byte window: 16 K rows of 256 bytes take 16 distinct
// chunks; 16 V^T rows of 128 bytes pair up by d & 1 and take 8 distinct
// units per parity. Every fragment address is a per-lane register plus an
// immediate.
// Staging goes straight from memory to LDS (buffer loads with the LDS
// destination bit, 16 bytes per lane): no registers, no vector ALU work and
// no LDS store instructions in the loop. Each lane picks the K chunk that
// belongs at its LDS slot, which applies the swizzle; V comes from the
// packing kernel already converted, transposed, reordered and swizzled, as
// one 64 x D tile image per (b, h, key tile) in the workspace (pack.hip),
// and is copied as is. K rows past the sequence read as zero. The loads for the
// tiles of the next step are issued at the top of a step and complete
// behind its computation; one barrier per tile. Causal: waves skip key tiles wholly
// above their own diagonal and mask only on the tiles that cross it;
// workgroups of one (b, h) are mapped to one XCD (shared L2 for their K/V
// stream), query blocks that see the most keys dispatched first.
//
// Lane layouts of v_mfma_f32_16x16x32_{bf16,f16} (checked on hardware):
//   A[i][k]: lane i + 16*(k/8), element k%8
//   B[k][j]: lane j + 16*(k/8), element k%8
//   C[i][j]: lane j + 16*(i/4), register i%4
#include "internal.h"
#include "mfma_common.h"

namespace parallax {
namespace {

using namespace mfma;

constexpr int kWaveRows = 16;      // query rows per wave

// LDS-DMA: global -> LDS, 16 bytes per lane at dst + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned short* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

// NW waves per workgroup (4: 64 query rows share each staged K/V tile).
template <int D, int NW, bool OUT_BF16>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_mfma_kernel(FwdParams p) {
  constexpr int kThreads = 64 * NW;
  constexpr int kBM = NW * kWaveRows;  // query rows per workgroup
  constexpr int NKB = kBN / 16;  // 16-key blocks of S^T per tile
  constexpr int NKS = kBN / 32;  // 32-key steps of O^T per tile
  constexpr int DT = D / 32;     // d-steps of S^T
  constexpr int DB = D / 16;     // 16-row blocks of O^T
  constexpr int CPR = D / 8;     // 16-byte chunks per K/V row
  constexpr int KPT = kBN * CPR / kThreads;  // tile rows each thread loads
  constexpr int KG = kBN / KPT;              // V staging: key groups
  constexpr int TILE = kBN * D;              // elements per K or V^T tile
  static_assert(KPT == 2 || KPT == 4, "tile load split");
  static_assert(kBN * CPR % kThreads == 0, "tile load split");

  __shared__ __attribute__((aligned(16))) unsigned short smem[2 * 2 * TILE];

  // ---- block -> (query block, h, b); one (b, h) stays on one XCD ----------
  // Workgroup i runs on XCD i % 8. With B*H a multiple of 8, (b, h) group g
  // goes to XCD g % 8, so every XCD gets the same heads of every sequence
  // (balanced also when packed sequences differ in length); otherwise the
  // XCDs take contiguous ranges of groups.
  const int nqb = (p.N + kBM - 1) / kBM;
  const int nbh = p.H * p.B;
  const int total = nqb * nbh;
  const int lin0 = blockIdx.x + nqb * (blockIdx.y + p.H * blockIdx.z);
  int qbl, bh;
  if ((nbh & 7) == 0) {
    const int slot = lin0 >> 3;
    qbl = slot % nqb;
    bh = (lin0 & 7) + 8 * (slot / nqb);
  } else {
    const int lin = (total & 7) == 0 ? (lin0 & 7) * (total >> 3) + (lin0 >> 3) : lin0;
    qbl = lin % nqb;
    bh = lin / nqb;
  }
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int qb = p.causal ? (nqb - 1 - qbl) : qbl;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lj = lane & 15;   // query (column) of this lane
  const int lg = lane >> 4;   // lane group 0..3
  const int q0 = qb * kBM;
  const int qw0 = q0 + wave * kWaveRows;
  const int qi = qw0 + lj;
  // Sequence b: N rows from row offset s0 (packed) or the b-th slice.
  int N = p.N;
  int64_t s0 = 0;
  if (p.cu_seqlens != nullptr) {
    const int a = p.cu_seqlens[b];
    const int e = p.cu_seqlens[b + 1];
    s0 = a;
    N = min(max(e - a, 0), p.N);
  }
  if (q0 >= N) return;   // whole workgroup past a shorter sequence's end
  const bool packed = p.cu_seqlens != nullptr;
  const int64_t bq = packed ? s0 * p.q_sn : (int64_t)b * p.q_sb;
  const int64_t br = packed ? s0 * p.r_sn : (int64_t)b * p.r_sb;
  const int64_t bk = packed ? s0 * p.k_sn : (int64_t)b * p.k_sb;
  const int64_t bo = packed ? s0 * p.o_sn : (int64_t)b * p.o_sb;
  const int bperm32 = (lane ^ 32) << 2;

  // ---- Q and R fragments: B operand of S^T and Rk^T ------------------------
  // A negative softmax scale is folded into Q (bf16 sign flip, exact) so the
  // kernel works with cs = |scale| * log2(e) > 0 and max(s) * cs = max(s*cs).
  // (clamped away from 0 so a masked logit of -inf stays -inf for scale 0)
  const float cs = fmaxf(fabsf(p.scale_log2), 1e-30f);
  const unsigned qsign = p.scale_log2 < 0.0f ? 0x80008000u : 0u;
  bf16x8_t qf[DT], rf[DT];
  {
    const int row = qi < N ? qi : N - 1;
    const char* qrow = reinterpret_cast<const char*>(p.q) +
                       (bq + (int64_t)row * p.q_sn + h * p.q_sh) * 2;
    const char* rrow = reinterpret_cast<const char*>(p.rho) +
                       (br + (int64_t)row * p.r_sn + h * p.r_sh) * 2;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(qrow + (32 * t + 8 * lg) * 2);
      const u32x4 c = *reinterpret_cast<const u32x4*>(rrow + (32 * t + 8 * lg) * 2);
      qf[t] = __builtin_bit_cast(bf16x8_t, qi < N ? (a ^ qsign) : z);
      rf[t] = __builtin_bit_cast(bf16x8_t, qi < N ? c : z);
    }
  }

  // ---- tile staging (global -> LDS, no registers) ---------------------------
  // Each wave issues KPT 1-KiB LDS-DMA loads per tile and buffer: lane L of
  // load blk = KPT*wave + i fills LDS bytes blk*1024 + 16*L.
  // K: that position holds row r = blk*RPK + L / CPR, chunk c' = L % CPR,
  //    i.e. global chunk c' ^ (r % CPR) of key row r (rows past N read 0).
  // V: the tile image written by the packing kernel is copied as is.
  constexpr int RPK = 512 / D;  // K rows per KiB
  const char* kbh = reinterpret_cast<const char*>(p.k) + (bk + h * p.k_sh) * 2;
  const int64_t kspan = (int64_t)(N - 1) * p.k_sn * 2 + D * 2;
  const int64_t kstep = (int64_t)kBN * p.k_sn * 2;
  const char* vtbh = reinterpret_cast<const char*>(p.vt) +
                     ((int64_t)(b * p.H + h) * p.vt_tiles) * (TILE * 2);
  int kdo[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int r = (KPT * wave + i) * RPK + lane / CPR;
    kdo[i] = r * (int)p.k_sn * 2 + (((lane % CPR) ^ (r % CPR)) << 4);
  }
  // LDS: [K buf 0][K buf 1][V^T buf 0][V^T buf 1]
  unsigned short* const sK0 = smem;
  unsigned short* const sV0 = smem + 2 * TILE;
  auto dma_k = [&](int it, unsigned short* dst) {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbh + it * kstep, kspan - it * kstep);
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      dma16(rk, dst + (KPT * wave + i) * 512, kdo[i]);
  };
  auto dma_v = [&](int it, unsigned short* dst) {
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(vtbh + (int64_t)it * (TILE * 2), (int64_t)(p.vt_tiles - it) * (TILE * 2));
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      dma16(rv, dst + (KPT * wave + i) * 512, (KPT * wave + i) * 1024 + lane * 16);
  };

  // LDS fragment offsets (elements within a tile); the 16-row block index
  // adds a compile-time constant.
  int kfo[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) kfo[t] = lj * D + (((4 * t + lg) ^ (lj % CPR)) << 3);
  int vfo[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    vfo[ks] = lj * kBN + (((4 * ks + lg) ^ ((lj >> 1) & 7)) << 3);

  // ---- state ----------------------------------------------------------------
  f32x4_t ov[DB], orv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    ov[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    orv[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float mref = -INFINITY;  // reference max (base-2), equal across a query's lanes
  float lsum = 0.0f, rsum = 0.0f;  // this lane's share of l and R
  // Shift of r = rho.k for this query (equal across its lanes): R and O_rv
  // accumulate r - cref. The output does not depend on the shift,
  // vbar (1 + rbar) - O_rv / l = vbar (1 + rbar - c) - (O_rv / l - c vbar),
  // but the fp16 operand p (r - cref) then carries the spread of r around
  // cref rather than r itself. cref is the softmax-weighted mean of r over
  // the first key tile (exact weights, fp32), fixed before the first
  // product; for the first 64 queries that is their exact rbar.
  float cref = 0.0f;

  int kend = N;
  if (p.causal) kend = (q0 + kBM < N) ? q0 + kBM : N;
  const int ntiles = (kend + kBN - 1) / kBN;
  const int wave_last_q = qw0 + kWaveRows - 1;
  // tiles [0, wtiles) carry keys this wave can see
  int wtiles = 0;
  if (qw0 < N) {
    const int wk = p.causal ? (wave_last_q + 1 < kend ? wave_last_q + 1 : kend) : kend;
    wtiles = (wk + kBN - 1) / kBN;
  }

  // S^T = K Q^T and Rk^T = K R^T - cref for one key tile held in LDS (the
  // shift enters as the accumulator's initial value).
  auto scores = [&](const unsigned short* kt, f32x4_t* s, f32x4_t* rk) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      rk[kb] = f32x4_t{-cref, -cref, -cref, -cref};
      bf16x8_t kf[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t)
        kf[t] = *reinterpret_cast<const bf16x8_t*>(kt + 16 * kb * D + kfo[t]);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t], qf[t], s[kb], 0, 0, 0);
        rk[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t], rf[t], rk[kb], 0, 0, 0);
      }
    }
  };

  // p = 2^(s*cs - mref - tau) and p*r as fp16 B operands of P V, with their
  // fp16-consistent sums; returns this lane's largest exponent
  // s*cs - mref - tau (masked keys give -inf).
  auto probs = [&](const f32x4_t* s, const f32x4_t* rk, f16x8_t* pf, f16x8_t* prf,
                   float& ls, float& rs) {
    const float nexp = -(mref + kTau);
    const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
    float xm = -INFINITY;
    ls = 0.0f;
    rs = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int kb = 2 * ks + (e >> 2);
        const int r = e & 3;
        const float x0 = fmaf(s[kb][r], cs, nexp);
        const float x1 = fmaf(s[kb][r + 1], cs, nexp);
        xm = fmaxf(xm, fmaxf(x0, x1));
        const float p0 = __builtin_amdgcn_exp2f(x0);
        const float p1 = __builtin_amdgcn_exp2f(x1);
        const f32x2_t pp = {p0, p1};
        const f32x2_t qq = {p0 * rk[kb][r], p1 * rk[kb][r + 1]};
        const f16x2_t ph = __builtin_convertvector(pp, f16x2_t);
        const f16x2_t qh = __builtin_convertvector(qq, f16x2_t);
        ls = __builtin_amdgcn_fdot2(ph, one2, ls, false);
        rs = __builtin_amdgcn_fdot2(qh, one2, rs, false);
        pf[ks][e] = ph[0];
        pf[ks][e + 1] = ph[1];
        prf[ks][e] = qh[0];
        prf[ks][e + 1] = qh[1];
      }
    return xm;
  };

  // Keys of tile j0 past the sequence or above the diagonal get s = -inf.
  // For (kb, r) this lane holds key j0 + 16*kb + 4*lg + r.
  auto mask_tile = [&](int j0, f32x4_t* s) {
    if ((p.causal && j0 + kBN - 1 > qw0) || j0 + kBN > N) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kj = j0 + 16 * kb + 4 * lg + r;
          if (kj >= N || (p.causal && kj > qi)) s[kb][r] = -INFINITY;
        }
    }
  };

  // The scores of the next tile and the probabilities of this one in one
  // straight-line block: the two are independent, so the exp / convert work
  // issues in the shadow of the matrix products. The order is pinned: the
  // K fragments of the first 16-key block up front, then per product up to
  // four vector instructions, with the next block's fragments read while
  // the current block's products run.
  auto scores_probs = [&](const unsigned short* kt, f32x4_t* s2, f32x4_t* rk2,
                          const f32x4_t* s, const f32x4_t* rk, f16x8_t* pf, f16x8_t* prf,
                          float& ls, float& rs) {
    scores(kt, s2, rk2);
    const float xm = probs(s, rk, pf, prf, ls, rs);
    __builtin_amdgcn_sched_group_barrier(0x100, DT, 0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        if (kb + 1 < NKB && i < DT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    return xm;
  };

  // O_v^T += V^T P^T and O_rv^T += V^T (P o Rk)^T with V^T of the tile in
  // LDS; each fragment is read four products ahead of its use.
  auto pv = [&](const unsigned short* vt, const f16x8_t* pf, const f16x8_t* prf) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f16x8_t vf = *reinterpret_cast<const f16x8_t*>(vt + 16 * db * kBN + vfo[ks]);
        ov[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[ks], ov[db], 0, 0, 0);
        orv[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, prf[ks], orv[db], 0, 0, 0);
      }
    constexpr int NV = NKS * DB;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (i + 4 < NV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // One tile j of this wave: (s, rk) hold its scores; the scores of tile
  // j+1 go to (sn, rn) from the K tile kn. Exponents are taken against the
  // current reference first; only if one of them is positive somewhere in
  // the wave (a key above mref + tau; on the first tile mref is -inf and
  // every exponent is +inf or NaN) are the four lanes of a query reduced to
  // the exact row max, the reference raised, the state rescaled and the
  // tile's probabilities recomputed.
  auto step = [&](int j, f32x4_t* s, const f32x4_t* rk, f32x4_t* sn, f32x4_t* rn,
                  const unsigned short* kn, const unsigned short* vt) {
    mask_tile(j * kBN, s);
    f16x8_t pf[NKS], prf[NKS];
    float ls, rs, xm;
    if (j + 1 < wtiles)
      xm = scores_probs(kn, sn, rn, s, rk, pf, prf, ls, rs);
    else
      xm = probs(s, rk, pf, prf, ls, rs);
    if (__builtin_expect(__any(xm > 0.0f), 0)) {
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        mloc = fmaxf(fmaxf(mloc, fmaxf(s[kb][0], s[kb][1])), fmaxf(s[kb][2], s[kb][3]));
      mloc *= cs;
      mloc = fmaxf(mloc, xor16(mloc));
      mloc = fmaxf(mloc, xor32(mloc, bperm32));
      const float mnew = fmaxf(mref, mloc);
      const float alpha = (mnew == mref) ? 1.0f : __builtin_amdgcn_exp2f(mref - mnew);
      mref = mnew;
      lsum *= alpha;
      rsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) { ov[i] *= alpha; orv[i] *= alpha; }
      probs(s, rk, pf, prf, ls, rs);
    }
    lsum += ls;
    rsum += rs;
    pv(vt, pf, prf);
  };

  // ---- pipeline -------------------------------------------------------------
  // Step j computes the scores of tile j+1 (K runs one tile ahead of V)
  // together with the softmax of tile j, then P V of tile j.
  // LDS at the start of step j: K(j+1) in K buf (j+1)&1, V(j) in V buf
  // j&1; during it K(j+2) and V(j+1) are staged into the other buffers.
  f32x4_t sa[NKB], ra[NKB], sb[NKB], rb[NKB];
  dma_k(0, sK0);
  dma_v(0, sV0);
  dma_k(1, sK0 + TILE);
  __syncthreads();                    // K(0), V(0), K(1) in LDS
  if (wtiles > 0) {
    scores(sK0, sa, ra);              // cref = 0: ra holds r itself
    // cref = weighted mean of r over tile 0 with the tile's exact softmax
    // weights, then tile 0's r moved to r - cref like every later tile's.
    mask_tile(0, sa);
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      mloc = fmaxf(fmaxf(mloc, fmaxf(sa[kb][0], sa[kb][1])), fmaxf(sa[kb][2], sa[kb][3]));
    mloc *= cs;
    mloc = fmaxf(mloc, xor16(mloc));
    mloc = fmaxf(mloc, xor32(mloc, bperm32));
    float sp = 0.0f, sr = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float w = __builtin_amdgcn_exp2f(fmaf(sa[kb][r], cs, -mloc));
        sp += w;
        sr = fmaf(w, ra[kb][r], sr);
      }
    sp += xor16(sp);
    sp += xor32(sp, bperm32);
    sr += xor16(sr);
    sr += xor32(sr, bperm32);
    cref = sp > 0.0f ? sr / sp : 0.0f;   // no visible key (mloc = -inf): 0
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) ra[kb][r] -= cref;
  }
  __syncthreads();                    // K buf 0 free again
  for (int j = 0; j < ntiles; j += 2) {
    // even tile j: K(j+1) in K buf 1, V(j) in V buf 0
    if (j + 2 < ntiles) dma_k(j + 2, sK0);
    if (j + 1 < ntiles) dma_v(j + 1, sV0 + TILE);
    if (j < wtiles) step(j, sa, ra, sb, rb, sK0 + TILE, sV0);
    __syncthreads();
    if (j + 1 >= ntiles) break;
    // odd tile j+1: K(j+2) in K buf 0, V(j+1) in V buf 1
    if (j + 3 < ntiles) dma_k(j + 3, sK0 + TILE);
    if (j + 2 < ntiles) dma_v(j + 2, sV0);
    if (j + 1 < wtiles) step(j + 1, sb, rb, sa, ra, sK0, sV0 + TILE);
    __syncthreads();
  }

  // ---- epilogue: combine the four lanes of each query, write ---------------
  float l = lsum + xor16(lsum);
  l += xor32(l, bperm32);
  float R = rsum + xor16(rsum);
  R += xor32(R, bperm32);
  if (qi < N) {
    const bool any = l > 0.0f;
    const float inv = any ? 1.0f / l : 0.0f;
    const int64_t obase = bo + (int64_t)qi * p.o_sn + h * p.o_sh;
    if (p.vbar != nullptr) {
      // training forward: keep vbar and {lse2, rbar} for the backward
      float* vb = p.vbar + (((int64_t)b * p.N + qi) * p.H + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4_t*>(vb + 16 * db + 4 * lg) = ov[db] * inv;
      if (lg == 0) {
        const f32x2_t lr = {mref + kTau + __log2f(l), cref + R * inv};
        *reinterpret_cast<f32x2_t*>(p.lse_rbar + 2 * (((int64_t)b * p.H + h) * p.N + qi)) = lr;
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 16 * db + 4 * lg;
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        o[r] = any ? finish(inv, R, ov[db][r], orv[db][r]) : 0.0f;
      if constexpr (OUT_BF16) {
        unsigned short* dst = reinterpret_cast<unsigned short*>(p.out) + obase + d;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r] = f32_to_bf16_bits(o[r]);
      } else {
        float* dst = reinterpret_cast<float*>(p.out) + obase + d;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r] = o[r];
      }
    }
  }
}

template <int D, int NW>
hipError_t launch_mfma(const FwdParams& p, bool out_bf16, hipStream_t stream) {
  constexpr int bm = NW * kWaveRows;
  PackParams pk{};
  pk.src = p.v;
  pk.sb = p.v_sb; pk.sn = p.v_sn; pk.sh = p.v_sh;
  pk.B = p.B; pk.N = p.N; pk.H = p.H;
  pk.dst = p.vt;
  pk.tiles = p.vt_tiles;
  pk.cu_seqlens = p.cu_seqlens;
  hipError_t e = launch_pack_t(pk, D, kBN, true, stream);
  if (e != hipSuccess) return e;
  const dim3 grid((p.N + bm - 1) / bm, p.H, p.B);
  if (out_bf16)
    hipLaunchKernelGGL((fwd_mfma_kernel<D, NW, true>), grid, dim3(64 * NW), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<D, NW, false>), grid, dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int D, bool out_bf16,
                           hipStream_t stream) {
  return D == 128 ? launch_mfma<128, 4>(p, out_bf16, stream)
                  : launch_mfma<64, 4>(p, out_bf16, stream);
}

}  // namespace parallax
