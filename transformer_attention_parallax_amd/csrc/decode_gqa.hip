// decode_gqa.hip -- Parallax attention decode with grouped query heads and
// an optional paged KV cache (bf16 inputs, gfx950 matrix cores).
//
// Same computation as decode.hip (one streaming pass over K and V feeds
// both the softmax branch and the covariance branch; zubnet.ai news item on
// Parallax, second paragraph), for G = Hq / Hkv query heads that share one
// key-value head, each with its own probe rho:
//   s_g(j) = scale q_g.k_j,  r_g(j) = rho_g.k_j,  p_g(j) = softmax_j(s_g),
//   o_g = vbar_g (1 + rbar_g) - sum_j p_g(j) r_g(j) v_j.
// One workgroup streams the keys of one (sequence, kv head, split) once for
// all G heads. Per 16-key tile the 2G dot products of every key are one
// dense product S^T = K [q_1..q_G, rho_1..rho_G]^T (16 x D by D x 16, the
// columns past 2G zero), and the 2G weighted sums over the keys are one
// product Out = W V with W = [p_1..p_G, p_1 r_1..p_G r_G]^T (16 x 16 by
// 16 x D): both run on the matrix cores, so the arithmetic per byte of
// K and V no longer grows with G on the vector ALUs.
//
// Layouts (v_mfma_f32_16x16x32_bf16 for S^T, v_mfma_f32_16x16x16_bf16 for
// Out; lane = c + 16 q with c = lane % 16, q = lane / 16):
//  * S^T output: lane (c, q) holds column c for keys 4q .. 4q+3, which is
//    exactly the A-operand layout of W in the second product: the weights
//    never move between lanes. Column G + c (r_c) takes p_c from lane c of
//    the same 16-lane row (DPP row shift by G).
//  * Out: lane (c, q) holds rows 4q .. 4q+3 (the weight columns) of d = c
//    in each 16-wide d block.
//
// K and V tiles reach LDS by buffer loads that write LDS directly (16 bytes
// per lane), so the bytes in flight cost no registers. Each wave streams its
// tiles through its own ring of NB buffers and waits on its own load
// counter. A workgroup takes one of two shapes (chosen by the host):
//  * nh kv heads of one sequence, one wave each (nh <= 8): every wave walks
//    all tiles of the split for its kv head, the waves in step (a barrier
//    per tile), so the rows that a paged cache keeps side by side for the kv
//    heads of one token are read at about the same time; each wave then
//    finishes its own kv head.
//  * one kv head, four waves: tile t of the split goes to wave t % 4, and
//    the four partial states are merged at the end (fewer split records
//    when there are few sequences).
// A tile's operands are read into registers as soon as it lands and
// its slot takes the next load before the tile's arithmetic, so NB tiles
// stay in flight while one is consumed. Rows are stored with their 16-byte
// chunks XOR-swizzled by the row index (one pattern for K, another for V),
// which keeps the K-operand reads (16 rows, one chunk each) and the
// transposing V reads (32 bytes of each of 8 rows per pass) free of bank
// conflicts.
//
// Online softmax in base-2 logits with a lazy reference: weights are
// 2^(x - m) with x = s log2(e); m moves (and the partial sums are rescaled)
// only when a key of the tile exceeds it by more than kTau, so weights stay
// below 2^kTau. Each weight enters the second product as the sum of two bf16
// numbers (hi = bf16(w), lo = bf16(w - hi): 16 significant bits, relative
// error below 2^-16), i.e. two products per d block; the row sums l and A_r
// are accumulated from the same hi + lo. V is bf16 already, so every product
// is exact and only the fp32 accumulation rounds.
//
// Paged cache: position l of sequence b lives in page block_table[b][l / P]
// at row l % P; element (page, t, hk, d) at page*kv_sb + t*kv_sl +
// hk*kv_sh + d. P is a multiple of 8, so the 4 (D = 128) or 8 (D = 64) rows
// one load instruction covers share a page. Keys whose page index falls
// outside [0, num_pages) are skipped: their slots are filled from page 0 and
// masked (weights and values set to zero). Without a block table the cache
// is contiguous, element (b, hk, l, d) at b*kv_sb + hk*kv_sh + l*kv_sl + d.
// Rows past the end of the split are loaded from its last row and masked.
//
// Split records [m, l, A_r, 0, A_v, A_rv] per (b, query head, split) are
// merged by the combine kernel of decode.hip.
#include "decode_common.h"

namespace parallax {
namespace {

using dec::f32_to_bf16_bits;
using dec::store_out;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTK = 16;             // keys per tile
constexpr int kMaxWaves = 8;        // waves per workgroup at most
constexpr float kTau = 8.0f;        // headroom (base-2) before a rescale
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, gfx9 data format
constexpr int kNonTemporal = 2;     // cache-policy operand of buffer loads: nt

// K tiles: 16-byte chunk c of LDS row r sits at slot c ^ swz(r), so the
// K-operand reads (16 rows, one chunk each) touch 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// V tiles are read only through the transposing LDS read, whose 32 lanes per
// pass take two adjacent chunks (32 bytes) of each of 8 consecutive rows:
// chunk c of row r sits at slot c ^ vswz(r), which sends the chunk pair of
// those 8 rows to 8 distinct 32-byte bank groups (D = 128: 256-byte rows;
// D = 64: 128-byte rows, two rows per 256 bytes of banks).
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

// Wait until at most N vector-memory instructions of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane, as a
// streaming (non-temporal) read: every byte of the cache is used once.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, kNonTemporal);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const unsigned short* base,
                                                      int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned short*>(base), (short)0,
                                           bytes, kRsrcWord3);
}

// The value operands of one tile, DB transposing LDS reads
// (ds_read_b64_tr_b16) from the LDS byte addresses a[], followed in the same
// block by a wait for every LDS read of the wave: the slot they read is
// refilled next, and no load is left in flight when the block ends. (As a
// builtin, the transposing read makes the compiler wait for the LDS-DMA
// loads of the next tiles too, which would leave one tile in flight.)
typedef int i32x2_t __attribute__((ext_vector_type(2)));
template <int DB>
__device__ __forceinline__ void tr_reads_wait(i32x2_t (&v)[DB], const unsigned (&a)[DB]) {
  if constexpr (DB == 8) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7])
        : "memory");
  } else {
    static_assert(DB == 4, "head dimension 64 or 128");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  }
}

// x of lane - S within each row of 16 lanes (lanes below S read 0).
template <int S>
__device__ __forceinline__ float from_left(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + S, 0xF, 0xF, true));
}

// x from lane ^ 16 and from lane ^ 32.
__device__ __forceinline__ float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
__device__ __forceinline__ float xor32(float x, int bperm_addr) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(bperm_addr, __float_as_int(x)));
}

template <int D, int G, int WPH, int NB, bool PAGED, bool SPLIT, bool OUT_BF16>
__global__ __launch_bounds__(64 * kMaxWaves) void decode_gqa_kernel(DecodeParams p) {
  constexpr int RB = 2 * D;             // bytes per row
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;        // rows per load instruction
  constexpr int IPT = kTK / RPI;        // load instructions per tile and tensor
  constexpr int NI = 2 * IPT;           // load instructions per tile (K and V)
  constexpr int TB = kTK * RB;          // bytes of one tensor's tile
  constexpr int BUF = 2 * TB;           // K tile, then V tile
  constexpr int DM = D / 32;            // products for S^T
  constexpr int DB = D / 16;            // products for Out
  constexpr int NC = 2 * G;             // used weight columns
  constexpr unsigned FULL = (1u << kTK) - 1u;
  static_assert(NI * (NB - 1) <= 63, "load counter range");
  static_assert((32 + 16 * D) * 4 <= NB * BUF, "merge state fits a wave's ring");
  // NB ring slots per wave (the launch sizes it: waves x NB x BUF bytes)
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // Shape: nh kv heads of one sequence per workgroup, WPH waves per kv head
  // (WPH = 1, or WPH = 4 with nh = 1); wave w serves kv head w / WPH of the
  // group and takes tiles w % WPH, w % WPH + WPH, ... of the split.
  constexpr int wph = WPH;
  const int nh = WPH == 1 ? p.gqa_nh : 1;
  const int ngroups = p.Hkv / nh;
  // Workgroup i runs on XCD i % 8. Linear order (b, head group, split) is
  // dealt out in eight contiguous ranges, one per XCD, so the workgroups of
  // one sequence (which share its pages) run side by side on one XCD.
  int split, hk, b;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = wave / wph;            // kv head within the group
  const int sub = wave - hl * wph;      // this wave's share of the tiles
  {
    const int n = (int)gridDim.x;
    const int id = (int)blockIdx.x;
    const int lin = (n % 8 == 0) ? (id % 8) * (n / 8) + id / 8 : id;
    split = lin % p.nsplit;
    hk = ((lin / p.nsplit) % ngroups) * nh + hl;
    b = lin / (p.nsplit * ngroups);
  }
  const int lane = threadIdx.x & 63;
  const int lc = lane & 15;
  const int lq = lane >> 4;
  const int bperm32 = (lane ^ 32) << 2;

  int len = p.Lmax;
  if (p.seqlens != nullptr) {
    const int sl = p.seqlens[b];
    len = sl < len ? sl : len;
  }
  if (len < 0) len = 0;
  const int j0 = split * p.chunk;
  int j1 = j0 + p.chunk;
  if (j1 > len) j1 = len;
  const int ntiles = j1 > j0 ? (j1 - j0 + kTK - 1) / kTK : 0;
  const int nmine = ntiles > sub ? (ntiles - sub + wph - 1) / wph : 0;

  // B operand of S^T: column c < G is q of query head hk*G + c, column
  // G + c its rho; lane (c, q) holds d = 32 m + 8 q .. + 7 of product m.
  bf16x8_t qf[DM];
  {
    const unsigned short* src = nullptr;
    if (lc < G)
      src = reinterpret_cast<const unsigned short*>(p.q) + b * p.q_sb +
            (int64_t)(hk * G + lc) * p.q_sh;
    else if (lc < NC)
      src = reinterpret_cast<const unsigned short*>(p.rho) + b * p.r_sb +
            (int64_t)(hk * G + lc - G) * p.r_sh;
#pragma unroll
    for (int m = 0; m < DM; ++m) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (src != nullptr) w = *reinterpret_cast<const u32x4*>(src + 32 * m + 8 * lq);
      qf[m] = __builtin_bit_cast(bf16x8_t, w);
    }
    // Retire these loads before the first tile load is issued: the wait
    // counter is in order, and a wait for them inside the loop would also
    // wait for every tile in flight.
#pragma unroll
    for (int m = 0; m < DM; ++m) asm volatile("" ::"v"(qf[m]));
  }

  const float cs = p.scale_log2;
  const unsigned short* kbase = reinterpret_cast<const unsigned short*>(p.k);
  const unsigned short* vbase = reinterpret_cast<const unsigned short*>(p.v);
  const int nrec = (RPI - 1) * (int)p.kv_sl * 2 + RB;
  const int nrec_tile = (kTK - 1) * (int)p.kv_sl * 2 + RB;
  const int rsub = lane / CPR;          // row within a load instruction
  const int csub = lane % CPR;          // chunk slot within the row
  const int64_t cbase = PAGED ? (int64_t)hk * p.kv_sh
                              : (int64_t)b * p.kv_sb + (int64_t)hk * p.kv_sh;
  // Block-table entries are read through the constant address space so that
  // they become scalar loads (a vector load here would order behind the
  // tile loads in flight).
  typedef const __attribute__((address_space(4))) int32_t* const_i32p;
  const_i32p bt = PAGED ? (const_i32p)(p.block_table + (int64_t)b * p.bt_sb) : nullptr;
  // page cursor (index into the block-table row, row in page) of the first
  // row of the next tile this wave issues
  int pq = 0, pr = 0, sq = 0, sr = 0;
  if constexpr (PAGED) {
    const int r0 = j0 + sub * kTK;
    pq = r0 / p.page;
    pr = r0 - pq * p.page;
    sq = (wph * kTK) / p.page;
    sr = wph * kTK - sq * p.page;
  }

  // Byte offsets of this lane's 16-byte chunk in load instruction i when a
  // whole tile is addressed from its first row (K and V swizzles).
  int koff_tile[IPT], voff_tile[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int r = i * RPI + rsub;
    koff_tile[i] = r * (int)p.kv_sl * 2 + ((csub ^ swz<D>(r)) << 4);
    voff_tile[i] = r * (int)p.kv_sl * 2 + ((csub ^ vswz<D>(r)) << 4);
  }

  // Issue the loads of this wave's tile `it` into ring slot `slot`; returns
  // the mask of its valid keys.
  auto issue = [&](int it, int slot) -> unsigned {
    const int row0 = j0 + (sub + it * wph) * kTK;
    const int nvalid = min(kTK, j1 - row0);
    char* kd = smem + (wave * NB + slot) * BUF;
    char* vd = kd + TB;
    unsigned mask = 0;
    if (nvalid == kTK && (!PAGED || pr + kTK <= p.page)) {
      // all 16 rows at kv_sl strides from one base
      int64_t off;
      mask = FULL;
      if constexpr (PAGED) {
        int pg = bt[pq];
        if (!(pg >= 0 && pg < p.num_pages)) {
          pg = 0;
          mask = 0;
        }
        off = (int64_t)pg * p.kv_sb + (int64_t)pr * p.kv_sl + cbase;
      } else {
        off = cbase + (int64_t)row0 * p.kv_sl;
      }
      const __amdgpu_buffer_rsrc_t rk = rsrc(kbase + off, nrec_tile);
      const __amdgpu_buffer_rsrc_t rv = rsrc(vbase + off, nrec_tile);
#pragma unroll
      for (int i = 0; i < IPT; ++i) dma16(rk, kd + i * 1024, koff_tile[i]);
#pragma unroll
      for (int i = 0; i < IPT; ++i) dma16(rv, vd + i * 1024, voff_tile[i]);
    } else {
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        // rows past the end re-read the last valid row of the tile
        const int ir = min(i * RPI, ((nvalid - 1) / RPI) * RPI);
        const int re = min(rsub, nvalid - 1 - ir);
        int64_t off;
        bool pv = true;
        if constexpr (PAGED) {
          int q = pq, rr = pr + ir;
          while (rr >= p.page) {
            rr -= p.page;
            ++q;
          }
          int pg = bt[q];
          pv = pg >= 0 && pg < p.num_pages;
          if (!pv) pg = 0;
          off = (int64_t)pg * p.kv_sb + (int64_t)rr * p.kv_sl + cbase;
        } else {
          off = cbase + (int64_t)(row0 + ir) * p.kv_sl;
        }
        const int roff = re * (int)p.kv_sl * 2;
        dma16(rsrc(kbase + off, nrec), kd + i * 1024, roff + ((csub ^ swz<D>(i * RPI + rsub)) << 4));
        dma16(rsrc(vbase + off, nrec), vd + i * 1024, roff + ((csub ^ vswz<D>(i * RPI + rsub)) << 4));
        if (pv) mask |= ((1u << RPI) - 1u) << (i * RPI);
      }
      if (nvalid < kTK) mask &= (1u << nvalid) - 1u;
    }
    if constexpr (PAGED) {
      pr += sr;
      pq += sq;
      if (pr >= p.page) {
        pr -= p.page;
        ++pq;
      }
    }
    return mask;
  };

  float mref = -INFINITY;   // reference of column lc (used for lc < G)
  float accw = 0.0f;        // rounded weights of column lc over this lane's keys
  f32x4_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Operands of the tile being consumed, read out of its ring slot so the
  // slot can be refilled before the tile's arithmetic: K fragments of S^T
  // (lane (c, q) of product m: row c, d = 32 m + 8 q .. + 7) and the value
  // operand of Out (lane (c, q) of product db: V[4 q + e][16 db + c],
  // e = 0..3). The latter comes from the transposing LDS read of gfx950
  // (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives as
  // its element e element i % 4 of the 8 bytes addressed by lane 4 e + i / 4,
  // so lane (j, q) addresses row 4 q + j / 4 at d = 16 db + 4 (j % 4) .. + 3.
  bf16x8_t kf[DM];
  s16x4_t vf[DB];
  int kro[DM], vro[DB];
#pragma unroll
  for (int m = 0; m < DM; ++m) kro[m] = lc * RB + (((4 * m + lq) ^ swz<D>(lc)) << 4);
  {
    const int r = 4 * lq + (lc >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vro[db] = TB + r * RB + (((2 * db + ((lc & 3) >> 1)) ^ vswz<D>(r)) << 4) + 8 * (lc & 1);
  }
  const unsigned lds0 =
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)(smem + wave * NB * BUF);
  auto fetch = [&](int slot) {
    const char* kb = smem + (wave * NB + slot) * BUF;
#pragma unroll
    for (int m = 0; m < DM; ++m) kf[m] = *reinterpret_cast<const bf16x8_t*>(kb + kro[m]);
    unsigned va[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = lds0 + slot * BUF + vro[db];
    i32x2_t vr[DB];
    tr_reads_wait<DB>(vr, va);
#pragma unroll
    for (int db = 0; db < DB; ++db) vf[db] = __builtin_bit_cast(s16x4_t, vr[db]);
  };

  auto compute = [&](unsigned mask) {
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < DM; ++m) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[m], qf[m], s, 0, 0, 0);
    bool ok[4];
    float x[4];
    bool need = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ok[e] = (mask >> (4 * lq + e)) & 1u;
      x[e] = s[e] * cs;
      need = need || (lc < G && ok[e] && x[e] - mref > kTau);
    }
    if (__builtin_expect(__any(need), 0)) {
      float tm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (lc < G && ok[e]) tm = fmaxf(tm, x[e]);
      tm = fmaxf(tm, xor16(tm));
      tm = fmaxf(tm, xor32(tm, bperm32));
      const float mnew = fmaxf(mref, tm);
      const float al = (mnew == mref) ? 1.0f : __builtin_amdgcn_exp2f(mref - mnew);
      mref = mnew;
      const float alr = from_left<G>(al);
      const float a = lc < G ? al : (lc < NC ? alr : 1.0f);
      accw *= a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(a, 4 * lq + r);   // factor of weight column 4q + r
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][r] *= ar;
      }
    }
    f32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pe = __builtin_amdgcn_exp2f(x[e] - mref);
      const float pl = from_left<G>(pe);
      const float we = lc < G ? pe : pl * s[e];
      w[e] = (ok[e] && lc < NC) ? we : 0.0f;
    }
    // w = hi + lo, both bf16: 16 significant bits reach the products
    const bf16x4_t whi = __builtin_convertvector(w, bf16x4_t);
    f32x4_t wr;
#pragma unroll
    for (int e = 0; e < 4; ++e) wr[e] = w[e] - (float)whi[e];
    const bf16x4_t wlo = __builtin_convertvector(wr, bf16x4_t);
#pragma unroll
    for (int e = 0; e < 4; ++e) accw += (float)whi[e] + (float)wlo[e];
    const s16x4_t wa = __builtin_bit_cast(s16x4_t, whi);
    const s16x4_t wb = __builtin_bit_cast(s16x4_t, wlo);
    // masked keys may hold anything (even NaN): their values are zeroed
    // (the mask is the same for the whole wave)
    if (mask != FULL) {
      const s16x4_t keep = {(short)(ok[0] ? -1 : 0), (short)(ok[1] ? -1 : 0),
                            (short)(ok[2] ? -1 : 0), (short)(ok[3] ? -1 : 0)};
#pragma unroll
      for (int db = 0; db < DB; ++db) vf[db] = vf[db] & keep;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wa, vf[db], acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wb, vf[db], acc[db], 0, 0, 0);
    }
  };

  // Ring of NB slots: tiles it .. it + NB - 1 are in flight when tile it is
  // waited for; its operands are then read into registers and its slot
  // takes tile it + NB before the arithmetic, so NB tiles stay in flight
  // while a tile is consumed. mq[k] is the key mask of tile it + k.
  unsigned mq[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) mq[u] = u < nmine ? issue(u, u) : 0u;
  int slot = 0;
  for (int it = 0; it < nmine; ++it) {
    if (it + NB - 1 < nmine)
      wait_vmem<NI * (NB - 1)>();
    else
      wait_vmem<0>();
    fetch(slot);
    const unsigned mcur = mq[0];
#pragma unroll
    for (int u = 0; u < NB - 1; ++u) mq[u] = mq[u + 1];
    mq[NB - 1] = 0u;
    if (it + NB < nmine) mq[NB - 1] = issue(it + NB, slot);
    // With one wave per kv head every wave walks the same tiles: the heads
    // of the group keep in step, so their rows of a page are read together.
    if constexpr (WPH == 1) __builtin_amdgcn_s_barrier();
    compute(mcur);
    slot = slot == NB - 1 ? 0 : slot + 1;
  }

  // Column sums over the four key quads.
  accw += xor16(accw);
  accw += xor32(accw, bperm32);

  // Output (or split record) of query head hkk * G + g, element d.
  auto emit = [&](int hkk, int g, int d, float M, float L, float AR, float AV, float ARV) {
    const int hq = hkk * G + g;
    if constexpr (SPLIT) {
      constexpr int REC = decode_record_floats(D);
      float* rec = p.ws + ((int64_t)(b * p.H + hq) * p.nsplit + split) * REC;
      if (d == 0) {
        rec[0] = M;
        rec[1] = L;
        rec[2] = AR;
        rec[3] = 0.0f;
      }
      rec[4 + d] = AV;
      rec[4 + D + d] = ARV;
    } else {
      store_out<OUT_BF16>(p.out, b * p.o_sb + hq * p.o_sh + d, dec::finish(L, AR, AV, ARV));
    }
  };
  // A wave's state in LDS, ST floats: reference m and column sums of the 16
  // weight columns, then the 16 x D weighted value sums.
  constexpr int ST = 32 + 16 * D;
  auto put_state = [&](float* st) {
    if (lq == 0) {
      st[lc] = mref;
      st[16 + lc] = accw;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[32 + (4 * lq + r) * D + 16 * db + lc] = acc[db][r];
  };

  if constexpr (WPH == 1) {
    // The wave alone holds its kv head's state: it passes it between its
    // lanes through its own ring slots (no other wave reads them).
    float* st = reinterpret_cast<float*>(smem + wave * NB * BUF);
    put_state(st);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the writes are done
    __builtin_amdgcn_wave_barrier();
    for (int idx = lane; idx < G * D; idx += 64) {
      const int g = idx / D;
      const int d = idx - g * D;
      const float M = st[g];
      float L = 0.0f, AR = 0.0f, AV = 0.0f, ARV = 0.0f;
      if (M != -INFINITY) {
        L = st[16 + g];
        AR = st[16 + G + g];
        AV = st[32 + g * D + d];
        ARV = st[32 + (G + g) * D + d];
      }
      emit(hk, g, d, M, L, AR, AV, ARV);
    }
    return;
  }

  // Merge the WPH wave states of the workgroup's one kv head.
  __syncthreads();
  float* st = reinterpret_cast<float*>(smem);   // wave w's state at w * ST
  put_state(st + wave * ST);
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * WPH) {
    const int g = idx / D;
    const int d = idx - g * D;
    const float* s0 = st;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPH; ++w) M = fmaxf(M, s0[w * ST + g]);
    float L = 0.0f, AR = 0.0f, AV = 0.0f, ARV = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WPH; ++w) {
        const float* sw = s0 + w * ST;
        const float mw = sw[g];
        const float wt = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        L = fmaf(wt, sw[16 + g], L);
        AR = fmaf(wt, sw[16 + G + g], AR);
        AV = fmaf(wt, sw[32 + g * D + d], AV);
        ARV = fmaf(wt, sw[32 + (G + g) * D + d], ARV);
      }
    }
    emit(hk, g, d, M, L, AR, AV, ARV);
  }
}

// Ring depth per wave: 16 KiB of LDS per wave, up to 128 KiB per workgroup.
template <int D>
constexpr int ring_depth() { return D == 128 ? 2 : 4; }

template <int D, int G, int WPH, bool PAGED>
hipError_t launch_w(const DecodeParams& p, bool out_bf16, hipStream_t stream) {
  constexpr int NB = ring_depth<D>();
  constexpr size_t BUF = 2 * kTK * 2 * D;
  const int nh = WPH == 1 ? p.gqa_nh : 1;
  const int nw = nh * WPH;
  const dim3 grid(p.nsplit * (p.Hkv / nh) * p.B);
  const dim3 block(64 * nw);
  const size_t lds = (size_t)nw * NB * BUF;
  if (p.nsplit > 1) {
    hipLaunchKernelGGL((decode_gqa_kernel<D, G, WPH, NB, PAGED, true, false>), grid, block, lds,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_combine(p, D, out_bf16, stream);
  }
  if (out_bf16)
    hipLaunchKernelGGL((decode_gqa_kernel<D, G, WPH, NB, PAGED, false, true>), grid, block, lds,
                       stream, p);
  else
    hipLaunchKernelGGL((decode_gqa_kernel<D, G, WPH, NB, PAGED, false, false>), grid, block,
                       lds, stream, p);
  return hipGetLastError();
}

template <int D, int G, bool PAGED>
hipError_t launch_g(const DecodeParams& p, bool out_bf16, hipStream_t stream) {
  return p.gqa_wph == 1 ? launch_w<D, G, 1, PAGED>(p, out_bf16, stream)
                        : launch_w<D, G, 4, PAGED>(p, out_bf16, stream);
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
  // shapes: nh (dividing Hkv, at most 8) kv heads of one wave each, or one
  // kv head of four waves
  if (!((p.gqa_wph == 1 && p.gqa_nh >= 1 && p.gqa_nh <= kMaxWaves && p.Hkv % p.gqa_nh == 0) ||
        (p.gqa_wph == 4 && p.gqa_nh == 1)))
    return hipErrorInvalidValue;
  const bool paged = p.block_table != nullptr;
  if (D == 128)
    return paged ? launch_d<128, true>(p, group, out_bf16, stream)
                 : launch_d<128, false>(p, group, out_bf16, stream);
  return paged ? launch_d<64, true>(p, group, out_bf16, stream)
               : launch_d<64, false>(p, group, out_bf16, stream);
}

}  // namespace parallax
