// api.hip -- the C ABI of libparallax: argument validation, split planning
// and kernel dispatch. Every check runs on the host before any HIP call.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "internal.h"
#include "parallax.h"

// Device scratch of parallax_decode_noalloc: the split records of one call
// (at most kScratchBytes). Every GPU the library runs on holds its own copy
// until the process ends. Host code never uses this name as an address: it
// takes each device's address once from hipGetSymbolAddress (scratch_on).
namespace {
constexpr size_t kScratchBytes = (size_t)4 << 20;
}
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_msg[512] = "";

parallax_status_t fail(parallax_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

parallax_status_t ok() {
  g_msg[0] = '\0';
  return PARALLAX_OK;
}

// Split planning for decode. The target counts workgroups for an MI355X:
// 256 compute units, several resident 256-thread workgroups each.
constexpr int kComputeUnits = 256;
constexpr int kSplitAlign = 64;        // split boundaries are multiples of this
constexpr int kMaxSplits = parallax::kMaxDecodeSplits;

// Automatic split choice: about `workgroups` workgroups in all, each split at
// least `min_keys` long, contexts shorter than `min_context` unsplit. Both
// decode kernels stream best with about one workgroup per CU; every split
// adds a record to merge and, when the context is split at all, a second
// launch. Measured (split counts swept from 1 to 64 per point, 16 heads /
// 32 query and 8 kv heads, D 128): MHA at batch 1 and 512 keys is fastest
// unsplit (11.6 us, 13.4 with 2 splits), at 2048 keys with 8 splits (13.7
// us, 15.7 with 4) and at 8192 and 32768 keys with 16; from batch 8 on one
// or two splits are within 4 % of the best. The grouped kernel has only 8
// kv-head streams per sequence and each workgroup streams its range through
// an LDS ring: at batch 1 it wants ranges down to 128 keys (2048 keys: 16
// splits 13.2 us, 4 splits 19.5 us; 8192 keys: 32 splits 16.8 us, 16
// splits 19.2 us).
struct SplitTarget {
  int workgroups;
  int min_keys;
  int min_context;   // shorter contexts are never split automatically
};
constexpr SplitTarget kMhaSplits{kComputeUnits, 256, 1024};
constexpr SplitTarget kGqaSplits{kComputeUnits, 128, 0};

struct SplitPlan {
  int nsplit;
  int chunk;
};

SplitPlan plan_splits(int B, int H, int Lmax, int requested,
                      SplitTarget tgt = kMhaSplits) {
  SplitPlan sp{1, Lmax > 0 ? Lmax : 1};
  if (Lmax <= 0) return sp;
  const int max_by_align = (Lmax + kSplitAlign - 1) / kSplitAlign;
  int s;
  if (requested > 0) {
    s = requested;
  } else {
    const long bh = (long)B * (long)H;
    s = 1;
    if (bh > 0 && bh < tgt.workgroups && Lmax >= tgt.min_context)
      s = (int)((tgt.workgroups + bh - 1) / bh);
    const int max_by_len = Lmax / tgt.min_keys;
    if (s > max_by_len) s = max_by_len;
  }
  if (s > max_by_align) s = max_by_align;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  // round the chunk up to the alignment, then drop splits left empty
  int chunk = (Lmax + s - 1) / s;
  chunk = ((chunk + kSplitAlign - 1) / kSplitAlign) * kSplitAlign;
  sp.chunk = chunk;
  sp.nsplit = (Lmax + chunk - 1) / chunk;
  return sp;
}

// Grouped-query decode: split plan and workgroup shape. A workgroup can
// hold nh kv heads of one sequence with one wave each (nh = the largest of
// 8, 4, 2, 1 dividing Hkv), the waves walking the same tiles in step, so a
// paged cache's rows of one page, which lie side by side for the kv heads
// of a token, are read together (a read-only probe of the token-major page
// pattern: 7.29 TB/s this way against 6.70 with each kv head in a workgroup
// of its own); its splits aim at 8 waves per CU. Otherwise a workgroup
// holds one kv head with 4 waves sharing its tiles, which fills the chip
// with fewer split records. Paged caches take the grouped shape once
// sequences x head groups x cache length reach kGqaGroupedMinKeys;
// contiguous caches (whose kv heads lie apart anyway) only when it needs no
// split. Measured (32 query / 8 kv heads, one box, grouped against one kv
// head per workgroup): paged 256 x 8192 1220 / 1332 us, 64 x 8192 321 /
// 356, 32 x 8192 166 / 177, 8 x 32768 169 / 181, 64 x 2048 equal, 8 x 8192
// 52 / 51, 1 x 8192 25 / 14.5; contiguous 256 x 2048 328 / 354, 256 x 8192
// 1219 / 1229, but 64 x 8192 332 / 320 and 8 x 32768 177 / 164. A paged
// cache with fewer than kGqaGroupedMinHeads kv heads per group keeps one kv
// head per workgroup: its token rows are too short for the joint read to
// pay. Measured (paged, 8192 keys, grouped against one kv head per
// workgroup, query / kv heads): 64 sequences 8 / 1 59.6 / 48.5 us, 24 / 3
// 160 / 145, 48 / 6 306 / 272; 128 sequences 16 / 2 180 / 169, but 32 / 4
// 345 / 360.
constexpr long kGqaGroupedMinKeys = 1L << 17;
constexpr int kGqaGroupedMinHeads = 4;
struct GqaPlan {
  SplitPlan sp;
  int nh, wph;
};
GqaPlan plan_gqa(int B, int Hkv, int Lmax, bool paged, int requested) {
  GqaPlan g{};
  int nh = 8;
  while (nh > 1 && Hkv % nh != 0) nh >>= 1;
  const long groups = Hkv / nh;
  const SplitTarget grouped{kComputeUnits * (8 / nh), kGqaSplits.min_keys, 0};
  const bool use = paged ? nh >= kGqaGroupedMinHeads &&
                               (long)B * groups * (Lmax > 0 ? Lmax : 1) >= kGqaGroupedMinKeys
                         : (long)B * groups >= grouped.workgroups;
  if (use) {
    g.nh = nh;
    g.wph = 1;
    g.sp = plan_splits(B, (int)groups, Lmax, requested, grouped);
  } else {
    g.nh = 1;
    g.wph = 4;
    g.sp = plan_splits(B, Hkv, Lmax, requested, kGqaSplits);
  }
  return g;
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool valid_dtype(parallax_dtype_t t) {
  return t == PARALLAX_F32 || t == PARALLAX_BF16;
}

int dtype_bytes(parallax_dtype_t t) { return t == PARALLAX_BF16 ? 2 : 4; }

parallax_status_t check_head_dim(int D) {
  if (D <= 0) return fail(PARALLAX_ERR_INVALID_ARG, "D must be positive (got %d)", D);
  if (D != 64 && D != 128)
    return fail(PARALLAX_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", D);
  return PARALLAX_OK;
}

// Input tensor: non-null, 16-byte aligned, strides non-negative and whole
// multiples of 16 bytes.
parallax_status_t check_input(const char* name, const void* p, int esize,
                              const int64_t* strides, int nstrides) {
  if (p == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, 16))
    return fail(PARALLAX_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
  for (int i = 0; i < nstrides; ++i) {
    if (strides[i] < 0)
      return fail(PARALLAX_ERR_INVALID_ARG, "%s has a negative stride", name);
    if ((strides[i] * esize) % 16 != 0)
      return fail(PARALLAX_ERR_UNSUPPORTED,
                  "%s stride %lld is not a multiple of 16 bytes", name,
                  (long long)strides[i]);
  }
  return PARALLAX_OK;
}

// Launch grids put the heads and the batch (or splits) in their y and z
// dimensions, at most 65535 each, and kernels number their workgroups with
// 32-bit integers.
parallax_status_t check_grid(int64_t x, int64_t y, int64_t z) {
  if (y > 65535 || z > 65535 || x * y * z > (int64_t)INT32_MAX)
    return fail(PARALLAX_ERR_UNSUPPORTED,
                "launch grid of %lld x %lld x %lld workgroups exceeds the device limits",
                (long long)x, (long long)y, (long long)z);
  return PARALLAX_OK;
}

parallax_status_t check_output(const void* p, int esize, const int64_t* strides,
                               int nstrides) {
  if (p == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "out is NULL");
  if (!aligned(p, (uintptr_t)esize))
    return fail(PARALLAX_ERR_UNSUPPORTED, "out is not %d-byte aligned", esize);
  for (int i = 0; i < nstrides; ++i)
    if (strides[i] < 0)
      return fail(PARALLAX_ERR_INVALID_ARG, "out has a negative stride");
  return PARALLAX_OK;
}

parallax_status_t from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PARALLAX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

extern "C" {

const char* parallax_status_string(parallax_status_t s) {
  switch (s) {
    case PARALLAX_OK: return "ok";
    case PARALLAX_ERR_INVALID_ARG: return "invalid argument";
    case PARALLAX_ERR_UNSUPPORTED: return "unsupported configuration";
    case PARALLAX_ERR_WORKSPACE: return "workspace missing or too small";
    case PARALLAX_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* parallax_last_error(void) { return g_msg; }

parallax_status_t parallax_decode_splits(int B, int H, int D, int Lmax,
                                         int num_splits, int* splits_out) {
  if (splits_out == nullptr)
    return fail(PARALLAX_ERR_INVALID_ARG, "splits_out is NULL");
  if (B < 0 || H < 0 || Lmax < 0 || num_splits < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "negative size or split count");
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  *splits_out = plan_splits(B, H, Lmax, num_splits).nsplit;
  return ok();
}

parallax_status_t parallax_decode_workspace_size(int B, int H, int D, int Lmax,
                                                 int num_splits, size_t* bytes) {
  if (bytes == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "bytes is NULL");
  int s = 0;
  parallax_status_t st = parallax_decode_splits(B, H, D, Lmax, num_splits, &s);
  if (st != PARALLAX_OK) return st;
  *bytes = s > 1 ? (size_t)B * (size_t)H * (size_t)s *
                       (size_t)parallax::decode_record_floats(D) * sizeof(float)
                 : 0;
  return ok();
}

}  // extern "C"

namespace {

// Device address of this device's scratch array, looked up once per device
// (with that device current) and kept; NULL after a failed lookup.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

parallax_status_t scratch_on(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(PARALLAX_ERR_HIP, "parallax_decode_noalloc: device of the stream: %s",
                hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PARALLAX_ERR_UNSUPPORTED, "parallax_decode_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess)
      return fail(PARALLAX_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(PARALLAX_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
      return fail(PARALLAX_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PARALLAX_OK;
}

// parallax_decode, and with noalloc set its variant whose split records
// live in this device's scratch array instead of a caller's workspace.
parallax_status_t decode_impl(
    const void* q, int64_t q_sb, int64_t q_sh, const void* rho, int64_t r_sb,
    int64_t r_sh, const void* k_cache, const void* v_cache, int64_t kv_sb,
    int64_t kv_sh, int64_t kv_sl, const int32_t* seqlens, void* out,
    int64_t o_sb, int64_t o_sh, int B, int H, int D, int Lmax, float scale,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype, int num_splits,
    void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  if (B < 0 || H < 0 || Lmax < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "negative size (B=%d H=%d Lmax=%d)", B, H, Lmax);
  if (num_splits < 0) return fail(PARALLAX_ERR_INVALID_ARG, "num_splits < 0");
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  if (!isfinite(scale)) return fail(PARALLAX_ERR_INVALID_ARG, "scale is not finite");
  if (B == 0 || H == 0) return ok();
  const int es = dtype_bytes(in_dtype);
  const int64_t qs[2] = {q_sb, q_sh}, rs[2] = {r_sb, r_sh};
  const int64_t kvs[3] = {kv_sb, kv_sh, kv_sl}, os[2] = {o_sb, o_sh};
  if ((st = check_input("q", q, es, qs, 2)) != PARALLAX_OK) return st;
  if (rho != nullptr && (st = check_input("rho", rho, es, rs, 2)) != PARALLAX_OK) return st;
  if (Lmax > 0) {
    if ((st = check_input("k_cache", k_cache, es, kvs, 3)) != PARALLAX_OK) return st;
    if ((st = check_input("v_cache", v_cache, es, kvs, 3)) != PARALLAX_OK) return st;
  }
  if ((st = check_output(out, dtype_bytes(out_dtype), os, 2)) != PARALLAX_OK) return st;
  if (seqlens != nullptr && !aligned(seqlens, 4))
    return fail(PARALLAX_ERR_UNSUPPORTED, "seqlens is not 4-byte aligned");

  const SplitPlan sp = plan_splits(B, H, Lmax, num_splits);
  if ((st = check_grid(sp.nsplit, H, B)) != PARALLAX_OK) return st;
  size_t need = 0;
  parallax_decode_workspace_size(B, H, D, Lmax, num_splits, &need);
  if (noalloc && need > 0) {
    if (need > kScratchBytes)
      return fail(PARALLAX_ERR_WORKSPACE,
                  "parallax_decode_noalloc: %d splits need %zu bytes of split records, "
                  "more than its %zu-byte device scratch (request fewer splits, or call "
                  "parallax_decode with a workspace)",
                  sp.nsplit, need, kScratchBytes);
    if ((st = scratch_on(static_cast<hipStream_t>(stream), &workspace)) != PARALLAX_OK)
      return st;
    workspace_bytes = kScratchBytes;
  }
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(PARALLAX_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s",
                  need, workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 16))
      return fail(PARALLAX_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  }

  parallax::DecodeParams p{};
  p.q = q;
  p.rho = rho;
  p.k = k_cache;
  p.v = v_cache;
  p.seqlens = seqlens;
  p.out = out;
  p.ws = static_cast<float*>(workspace);
  p.q_sb = q_sb; p.q_sh = q_sh; p.r_sb = r_sb; p.r_sh = r_sh;
  p.kv_sb = kv_sb; p.kv_sh = kv_sh; p.kv_sl = kv_sl;
  p.o_sb = o_sb; p.o_sh = o_sh;
  p.B = B; p.H = H; p.Lmax = Lmax;
  p.nsplit = sp.nsplit;
  p.chunk = sp.chunk;
  p.scale_log2 = scale * kLog2e;
  return from_hip(parallax::launch_decode(p, D, in_dtype == PARALLAX_BF16,
                                          out_dtype == PARALLAX_BF16,
                                          static_cast<hipStream_t>(stream)),
                  noalloc ? "parallax_decode_noalloc launch" : "parallax_decode launch");
}

}  // namespace

extern "C" {

parallax_status_t parallax_decode(
    const void* q, int64_t q_sb, int64_t q_sh, const void* rho, int64_t r_sb,
    int64_t r_sh, const void* k_cache, const void* v_cache, int64_t kv_sb,
    int64_t kv_sh, int64_t kv_sl, const int32_t* seqlens, void* out,
    int64_t o_sb, int64_t o_sh, int B, int H, int D, int Lmax, float scale,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype, int num_splits,
    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, q_sb, q_sh, rho, r_sb, r_sh, k_cache, v_cache, kv_sb, kv_sh, kv_sl,
                     seqlens, out, o_sb, o_sh, B, H, D, Lmax, scale, in_dtype, out_dtype,
                     num_splits, workspace, workspace_bytes, stream, false);
}

parallax_status_t parallax_decode_noalloc(
    const void* q, int64_t q_sb, int64_t q_sh, const void* rho, int64_t r_sb,
    int64_t r_sh, const void* k_cache, const void* v_cache, int64_t kv_sb,
    int64_t kv_sh, int64_t kv_sl, const int32_t* seqlens, void* out,
    int64_t o_sb, int64_t o_sh, int B, int H, int D, int Lmax, float scale,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype, int num_splits,
    void* stream) {
  return decode_impl(q, q_sb, q_sh, rho, r_sb, r_sh, k_cache, v_cache, kv_sb, kv_sh, kv_sl,
                     seqlens, out, o_sb, o_sh, B, H, D, Lmax, scale, in_dtype, out_dtype,
                     num_splits, nullptr, 0, stream, true);
}

parallax_status_t parallax_fwd_workspace_size(int B, int N, int H, int D,
                                              parallax_dtype_t in_dtype,
                                              size_t* bytes) {
  if (bytes == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 0 || N < 0 || H < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "negative size (B=%d N=%d H=%d)", B, N, H);
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  if (!valid_dtype(in_dtype)) return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  const size_t tiles = (size_t)((N + 63) / 64);
  *bytes = in_dtype == PARALLAX_BF16
               ? (size_t)B * (size_t)H * tiles *
                     (size_t)parallax::fwd_tile_elems(D) * sizeof(uint16_t)
               : 0;
  return ok();
}

}  // extern "C"

namespace {

// parallax_fwd, and with vbar / lse_rbar set the training forward.
parallax_status_t fwd_impl(
    const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
    int64_t k_sb, int64_t k_sn, int64_t k_sh, const void* v, int64_t v_sb,
    int64_t v_sn, int64_t v_sh, const void* rho, int64_t r_sb, int64_t r_sn,
    int64_t r_sh, void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh, int B,
    int N, int H, int D, float scale, int causal, parallax_dtype_t in_dtype,
    parallax_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
    void* stream, float* vbar, float* lse_rbar) {
  if (B < 0 || N < 0 || H < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "negative size (B=%d N=%d H=%d)", B, N, H);
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  if (!isfinite(scale)) return fail(PARALLAX_ERR_INVALID_ARG, "scale is not finite");
  if (B == 0 || N == 0 || H == 0) return ok();
  const int es = dtype_bytes(in_dtype);
  const int64_t qs[3] = {q_sb, q_sn, q_sh}, ks[3] = {k_sb, k_sn, k_sh};
  const int64_t vs[3] = {v_sb, v_sn, v_sh}, rs[3] = {r_sb, r_sn, r_sh};
  const int64_t os[3] = {o_sb, o_sn, o_sh};
  if ((st = check_input("q", q, es, qs, 3)) != PARALLAX_OK) return st;
  if ((st = check_input("k", k, es, ks, 3)) != PARALLAX_OK) return st;
  if ((st = check_input("v", v, es, vs, 3)) != PARALLAX_OK) return st;
  if ((st = check_input("rho", rho, es, rs, 3)) != PARALLAX_OK) return st;
  if ((st = check_output(out, dtype_bytes(out_dtype), os, 3)) != PARALLAX_OK) return st;
  if ((st = check_grid((N + 15) / 16, H, B)) != PARALLAX_OK) return st;

  if (in_dtype == PARALLAX_BF16) {
    // The matrix-core kernel addresses each (b, h) slice of K and V with
    // 32-bit buffer offsets.
    const int64_t sn = k_sn > v_sn ? k_sn : v_sn;
    const int64_t rows = N > 64 ? N : 64;
    if (sn * 2 * rows + 2 * D > 0x7fffffffLL)
      return fail(PARALLAX_ERR_UNSUPPORTED,
                  "bf16 prefill: one (b, h) slice of K or V spans more than 2 GiB");
  }
  size_t need = 0;
  parallax_fwd_workspace_size(B, N, H, D, in_dtype, &need);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(PARALLAX_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s",
                  need, workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 16))
      return fail(PARALLAX_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  }

  parallax::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.rho = rho; p.out = out;
  p.q_sb = q_sb; p.q_sn = q_sn; p.q_sh = q_sh;
  p.k_sb = k_sb; p.k_sn = k_sn; p.k_sh = k_sh;
  p.v_sb = v_sb; p.v_sn = v_sn; p.v_sh = v_sh;
  p.r_sb = r_sb; p.r_sn = r_sn; p.r_sh = r_sh;
  p.o_sb = o_sb; p.o_sn = o_sn; p.o_sh = o_sh;
  p.B = B; p.N = N; p.H = H;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;
  p.vt = static_cast<unsigned short*>(workspace);
  p.vt_tiles = (N + 63) / 64;
  p.vbar = vbar;
  p.lse_rbar = lse_rbar;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool ob = out_dtype == PARALLAX_BF16;
  if (in_dtype == PARALLAX_BF16)
    return from_hip(parallax::launch_fwd_bf16(p, D, ob, s), "parallax_fwd launch");
  // fp32: every query row is one stream of the decode kernel over its
  // sequence's keys (causal: the keys up to the row), B * N * H workgroups
  // of 256 threads with 16-byte loads of K and V rows that the rows of a
  // sequence share through L2. Measured faster than the tiled kernel at
  // every size tried (B1 N256 H2 D64: 7.6 against 72.5 us; B2 N2048 H16
  // D64: 1.94 against 2.51 ms). The decode kernel reads K and V with one
  // set of strides, and the grid holds B * N rows in its z dimension;
  // otherwise the tiled kernel runs.
  if (k_sb == v_sb && k_sn == v_sn && k_sh == v_sh && (int64_t)B * N <= 65535) {
    parallax::DecodeParams d{};
    d.q = q; d.rho = rho; d.k = k; d.v = v; d.out = out;
    d.q_sb = q_sb; d.q_sh = q_sh; d.q_sn = q_sn;
    d.r_sb = r_sb; d.r_sh = r_sh; d.r_sn = r_sn;
    d.kv_sb = k_sb; d.kv_sh = k_sh; d.kv_sl = k_sn;
    d.o_sb = o_sb; d.o_sh = o_sh; d.o_sn = o_sn;
    d.B = B * N; d.H = H; d.Lmax = N;
    d.nsplit = 1; d.chunk = N;
    d.scale_log2 = p.scale_log2;
    d.rows = N;
    d.causal_rows = causal ? 1 : 0;
    return from_hip(parallax::launch_decode(d, D, false, ob, s), "parallax_fwd launch");
  }
  return from_hip(parallax::launch_fwd_f32(p, D, ob, s), "parallax_fwd launch");
}

}  // namespace

extern "C" {

parallax_status_t parallax_fwd(
    const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
    int64_t k_sb, int64_t k_sn, int64_t k_sh, const void* v, int64_t v_sb,
    int64_t v_sn, int64_t v_sh, const void* rho, int64_t r_sb, int64_t r_sn,
    int64_t r_sh, void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh, int B,
    int N, int H, int D, float scale, int causal, parallax_dtype_t in_dtype,
    parallax_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
    void* stream) {
  return fwd_impl(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, v, v_sb, v_sn, v_sh, rho, r_sb,
                  r_sn, r_sh, out, o_sb, o_sn, o_sh, B, N, H, D, scale, causal, in_dtype,
                  out_dtype, workspace, workspace_bytes, stream, nullptr, nullptr);
}

parallax_status_t parallax_fwd_train(
    const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
    int64_t k_sb, int64_t k_sn, int64_t k_sh, const void* v, int64_t v_sb,
    int64_t v_sn, int64_t v_sh, const void* rho, int64_t r_sb, int64_t r_sn,
    int64_t r_sh, void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh, float* vbar,
    float* lse_rbar, int B, int N, int H, int D, float scale, int causal,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (valid_dtype(in_dtype) && in_dtype != PARALLAX_BF16)
    return fail(PARALLAX_ERR_UNSUPPORTED, "parallax_fwd_train supports bf16 inputs only");
  if (B > 0 && N > 0 && H > 0) {
    if (vbar == nullptr || lse_rbar == nullptr)
      return fail(PARALLAX_ERR_INVALID_ARG, "vbar or lse_rbar is NULL");
    if (!aligned(vbar, 16) || !aligned(lse_rbar, 8))
      return fail(PARALLAX_ERR_UNSUPPORTED,
                  "vbar must be 16-byte and lse_rbar 8-byte aligned");
  }
  return fwd_impl(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, v, v_sb, v_sn, v_sh, rho, r_sb,
                  r_sn, r_sh, out, o_sb, o_sn, o_sh, B, N, H, D, scale, causal, in_dtype,
                  out_dtype, workspace, workspace_bytes, stream, vbar, lse_rbar);
}

parallax_status_t parallax_fwd_varlen(
    const void* q, int64_t q_sn, int64_t q_sh, const void* k, int64_t k_sn, int64_t k_sh,
    const void* v, int64_t v_sn, int64_t v_sh, const void* rho, int64_t r_sn,
    int64_t r_sh, void* out, int64_t o_sn, int64_t o_sh, const int32_t* cu_seqlens,
    int B, int max_seqlen, int H, int D, float scale, int causal,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (B < 0 || max_seqlen < 0 || H < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "negative size (B=%d max_seqlen=%d H=%d)", B,
                max_seqlen, H);
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  if (in_dtype != PARALLAX_BF16)
    return fail(PARALLAX_ERR_UNSUPPORTED, "parallax_fwd_varlen supports bf16 inputs only");
  if (!isfinite(scale)) return fail(PARALLAX_ERR_INVALID_ARG, "scale is not finite");
  if (cu_seqlens == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (!aligned(cu_seqlens, 4))
    return fail(PARALLAX_ERR_UNSUPPORTED, "cu_seqlens is not 4-byte aligned");
  if (B == 0 || max_seqlen == 0 || H == 0) return ok();
  const int64_t qs[2] = {q_sn, q_sh}, ks[2] = {k_sn, k_sh}, vs[2] = {v_sn, v_sh};
  const int64_t rs[2] = {r_sn, r_sh}, os[2] = {o_sn, o_sh};
  if ((st = check_input("q", q, 2, qs, 2)) != PARALLAX_OK) return st;
  if ((st = check_input("k", k, 2, ks, 2)) != PARALLAX_OK) return st;
  if ((st = check_input("v", v, 2, vs, 2)) != PARALLAX_OK) return st;
  if ((st = check_input("rho", rho, 2, rs, 2)) != PARALLAX_OK) return st;
  if ((st = check_output(out, dtype_bytes(out_dtype), os, 2)) != PARALLAX_OK) return st;
  if ((st = check_grid((max_seqlen + 15) / 16, H, B)) != PARALLAX_OK) return st;
  {
    // one sequence's rows of K or V are addressed with 32-bit buffer offsets
    const int64_t sn = k_sn > v_sn ? k_sn : v_sn;
    const int64_t rows = max_seqlen > 64 ? max_seqlen : 64;
    if (sn * 2 * rows + 2 * D > 0x7fffffffLL)
      return fail(PARALLAX_ERR_UNSUPPORTED,
                  "bf16 prefill: one sequence of K or V spans more than 2 GiB");
  }
  size_t need = 0;
  parallax_fwd_workspace_size(B, max_seqlen, H, D, in_dtype, &need);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PARALLAX_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (!aligned(workspace, 16))
    return fail(PARALLAX_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");

  parallax::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.rho = rho; p.out = out;
  p.q_sn = q_sn; p.q_sh = q_sh; p.k_sn = k_sn; p.k_sh = k_sh;
  p.v_sn = v_sn; p.v_sh = v_sh; p.r_sn = r_sn; p.r_sh = r_sh;
  p.o_sn = o_sn; p.o_sh = o_sh;
  p.B = B; p.N = max_seqlen; p.H = H;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;
  p.vt = static_cast<unsigned short*>(workspace);
  p.vt_tiles = (max_seqlen + 63) / 64;
  p.cu_seqlens = cu_seqlens;
  return from_hip(parallax::launch_fwd_bf16(p, D, out_dtype == PARALLAX_BF16,
                                            static_cast<hipStream_t>(stream)),
                  "parallax_fwd_varlen launch");
}

parallax_status_t parallax_project(const void* x, int64_t x_st, const void* w, int64_t w_st,
                                   void* y, int64_t y_st, int M, int N, int K,
                                   parallax_dtype_t dtype, void* stream) {
  if (M < 0 || N < 0 || K < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "negative size (M=%d N=%d K=%d)", M, N, K);
  if (!valid_dtype(dtype)) return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  if (dtype != PARALLAX_BF16)
    return fail(PARALLAX_ERR_UNSUPPORTED, "parallax_project supports bf16 only");
  if (N % 256 != 0 || K % 64 != 0 || K == 0)
    return fail(PARALLAX_ERR_UNSUPPORTED,
                "N=%d must be a multiple of 256 and K=%d a positive multiple of 64", N, K);
  if (M == 0 || N == 0) return ok();
  parallax_status_t st;
  const int64_t xs[1] = {x_st}, ws[1] = {w_st}, ys[1] = {y_st};
  if ((st = check_input("x", x, 2, xs, 1)) != PARALLAX_OK) return st;
  if ((st = check_input("w", w, 2, ws, 1)) != PARALLAX_OK) return st;
  if (y == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "y is NULL");
  if (!aligned(y, 16) || y_st < 0 || (y_st * 2) % 16 != 0)
    return fail(PARALLAX_ERR_UNSUPPORTED, "y must be 16-byte aligned with 16-byte row stride");
  if (x_st < K || w_st < K || y_st < N)
    return fail(PARALLAX_ERR_INVALID_ARG, "row strides shorter than the rows");
  // a block's 256 rows of x or w are addressed with 32-bit offsets
  if (x_st > 0x7fffffffLL / 512 || w_st > 0x7fffffffLL / 512)
    return fail(PARALLAX_ERR_UNSUPPORTED, "row stride too large");
  parallax::ProjParams p{};
  p.x = x; p.x_st = x_st; p.w = w; p.w_st = w_st; p.y = y; p.y_st = y_st;
  p.M = M; p.N = N; p.K = K;
  return from_hip(parallax::launch_proj(p, static_cast<hipStream_t>(stream)),
                  "parallax_project launch");
}

parallax_status_t parallax_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                                       void* stream) {
  if (sink == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "sink is NULL");
  if (bytes < 0) return fail(PARALLAX_ERR_INVALID_ARG, "negative size");
  if (bytes > 0 && src == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "src is NULL");
  if (bytes % 16 != 0)
    return fail(PARALLAX_ERR_UNSUPPORTED, "size %lld is not a multiple of 16",
                (long long)bytes);
  if (!aligned(src, 16) || !aligned(sink, 4))
    return fail(PARALLAX_ERR_UNSUPPORTED, "src must be 16-byte and sink 4-byte aligned");
  return from_hip(parallax::launch_stream_read(src, bytes, sink,
                                               static_cast<hipStream_t>(stream)),
                  "parallax_stream_read launch");
}

parallax_status_t parallax_decode_gqa_splits(int B, int Hq, int Hkv, int D, int Lmax,
                                            int paged, int num_splits, int* splits_out) {
  if (splits_out == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "splits_out is NULL");
  if (B < 0 || Hq < 0 || Hkv <= 0 || Lmax < 0 || num_splits < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "bad size (B=%d Hq=%d Hkv=%d Lmax=%d)", B, Hq,
                Hkv, Lmax);
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  *splits_out = plan_gqa(B, Hkv, Lmax, paged != 0, num_splits).sp.nsplit;
  return ok();
}

parallax_status_t parallax_decode_gqa_workspace_size(int B, int Hq, int Hkv, int D,
                                                    int Lmax, int paged, int num_splits,
                                                    size_t* bytes) {
  if (bytes == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 0 || Hq < 0 || Hkv <= 0 || Lmax < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "bad size (B=%d Hq=%d Hkv=%d Lmax=%d)", B, Hq,
                Hkv, Lmax);
  if (num_splits < 0) return fail(PARALLAX_ERR_INVALID_ARG, "num_splits < 0");
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  const SplitPlan sp = plan_gqa(B, Hkv, Lmax, paged != 0, num_splits).sp;
  *bytes = sp.nsplit > 1 ? (size_t)B * (size_t)Hq * (size_t)sp.nsplit *
                               (size_t)parallax::decode_record_floats(D) * sizeof(float)
                         : 0;
  return ok();
}

parallax_status_t parallax_decode_gqa(
    const void* q, int64_t q_sb, int64_t q_sh, const void* rho, int64_t r_sb,
    int64_t r_sh, const void* k_cache, const void* v_cache, int64_t kv_sb,
    int64_t kv_sh, int64_t kv_sl, const int32_t* block_table, int64_t bt_sb,
    int page_size, int num_pages, const int32_t* seqlens, void* out, int64_t o_sb,
    int64_t o_sh, int B, int Hq, int Hkv, int D, int Lmax, float scale,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype, int num_splits,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || Lmax < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "bad size (B=%d Hq=%d Hkv=%d Lmax=%d)", B, Hq,
                Hkv, Lmax);
  if (Hq % Hkv != 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int group = Hq / Hkv;
  if (Hq > 0 && group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PARALLAX_ERR_UNSUPPORTED, "query heads per kv head %d (1, 2, 4 or 8)", group);
  if (num_splits < 0) return fail(PARALLAX_ERR_INVALID_ARG, "num_splits < 0");
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  if (in_dtype != PARALLAX_BF16)
    return fail(PARALLAX_ERR_UNSUPPORTED, "parallax_decode_gqa supports bf16 inputs only");
  if (!isfinite(scale)) return fail(PARALLAX_ERR_INVALID_ARG, "scale is not finite");
  if (block_table != nullptr) {
    if (page_size <= 0 || page_size % 8 != 0)
      return fail(PARALLAX_ERR_UNSUPPORTED, "page_size %d (a positive multiple of 8)",
                  page_size);
    if (num_pages <= 0) return fail(PARALLAX_ERR_INVALID_ARG, "num_pages %d", num_pages);
    if (seqlens == nullptr)
      return fail(PARALLAX_ERR_INVALID_ARG, "a paged cache needs seqlens");
    if (bt_sb < 0) return fail(PARALLAX_ERR_INVALID_ARG, "negative block table stride");
    if (!aligned(block_table, 4))
      return fail(PARALLAX_ERR_UNSUPPORTED, "block_table is not 4-byte aligned");
  }
  if (B == 0 || Hq == 0) return ok();
  const int64_t qs[2] = {q_sb, q_sh}, rs[2] = {r_sb, r_sh};
  const int64_t kvs[3] = {kv_sb, kv_sh, kv_sl}, os[2] = {o_sb, o_sh};
  if ((st = check_input("q", q, 2, qs, 2)) != PARALLAX_OK) return st;
  if ((st = check_input("rho", rho, 2, rs, 2)) != PARALLAX_OK) return st;
  if (Lmax > 0) {
    if ((st = check_input("k_cache", k_cache, 2, kvs, 3)) != PARALLAX_OK) return st;
    if ((st = check_input("v_cache", v_cache, 2, kvs, 3)) != PARALLAX_OK) return st;
  }
  if ((st = check_output(out, dtype_bytes(out_dtype), os, 2)) != PARALLAX_OK) return st;
  if (seqlens != nullptr && !aligned(seqlens, 4))
    return fail(PARALLAX_ERR_UNSUPPORTED, "seqlens is not 4-byte aligned");

  // one tile spans 16 rows of the cache from a 32-bit offset
  if (Lmax > 0 && (kv_sl > (int64_t)(INT32_MAX / 32) - D))
    return fail(PARALLAX_ERR_UNSUPPORTED, "kv row stride %lld is too large",
                (long long)kv_sl);
  const bool paged = block_table != nullptr;
  const GqaPlan gp = plan_gqa(B, Hkv, Lmax, paged, num_splits);
  const SplitPlan sp = gp.sp;
  if ((st = check_grid((int64_t)sp.nsplit * (Hkv / gp.nh) * B, 1, 1)) != PARALLAX_OK) return st;
  size_t need = 0;
  parallax_decode_gqa_workspace_size(B, Hq, Hkv, D, Lmax, paged ? 1 : 0, num_splits, &need);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(PARALLAX_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s",
                  need, workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 16))
      return fail(PARALLAX_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  }
  parallax::DecodeParams p{};
  p.q = q; p.rho = rho; p.k = k_cache; p.v = v_cache;
  p.seqlens = seqlens;
  p.out = out;
  p.ws = static_cast<float*>(workspace);
  p.q_sb = q_sb; p.q_sh = q_sh; p.r_sb = r_sb; p.r_sh = r_sh;
  p.kv_sb = kv_sb; p.kv_sh = kv_sh; p.kv_sl = kv_sl;
  p.o_sb = o_sb; p.o_sh = o_sh;
  p.B = B; p.H = Hq; p.Lmax = Lmax;
  p.nsplit = sp.nsplit;
  p.chunk = sp.chunk;
  p.scale_log2 = scale * kLog2e;
  p.Hkv = Hkv;
  p.block_table = block_table;
  p.bt_sb = bt_sb;
  p.page = page_size;
  p.num_pages = num_pages;
  p.gqa_nh = gp.nh;
  p.gqa_wph = gp.wph;
  return from_hip(parallax::launch_decode_gqa(p, D, group, out_dtype == PARALLAX_BF16,
                                              static_cast<hipStream_t>(stream)),
                  "parallax_decode_gqa launch");
}

namespace {

// Workspace of parallax_bwd: the per-query statistics, [B][H][N] float4.
size_t bwd_workspace_bytes(int B, int N, int H) {
  return ((size_t)B * (size_t)H * (size_t)N * 16 + 255) & ~(size_t)255;
}

}  // namespace

parallax_status_t parallax_bwd_workspace_size(int B, int N, int H, int D,
                                              parallax_dtype_t in_dtype,
                                              size_t* bytes) {
  if (bytes == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 0 || N < 0 || H < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "negative size (B=%d N=%d H=%d)", B, N, H);
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  if (!valid_dtype(in_dtype)) return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  if (in_dtype != PARALLAX_BF16)
    return fail(PARALLAX_ERR_UNSUPPORTED, "parallax_bwd supports bf16 inputs only");
  *bytes = (B == 0 || N == 0 || H == 0) ? 0 : bwd_workspace_bytes(B, N, H);
  return ok();
}

}  // extern "C"

namespace {

// A training forward's saved tensors (parallax_bwd_saved).
struct SavedFwd {
  const void* out;
  int64_t o_sb, o_sn, o_sh;
  bool out_bf16;
  const float* vbar;
  const float* lse_rbar;
};

parallax_status_t bwd_impl(
    const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
    int64_t k_sb, int64_t k_sn, int64_t k_sh, const void* v, int64_t v_sb,
    int64_t v_sn, int64_t v_sh, const void* rho, int64_t r_sb, int64_t r_sn,
    int64_t r_sh, const void* dout, int64_t g_sb, int64_t g_sn, int64_t g_sh,
    float* dq, int64_t dq_sb, int64_t dq_sn, int64_t dq_sh, float* dk,
    int64_t dk_sb, int64_t dk_sn, int64_t dk_sh, float* dv, int64_t dv_sb,
    int64_t dv_sn, int64_t dv_sh, float* drho, int64_t dr_sb, int64_t dr_sn,
    int64_t dr_sh, int B, int N, int H, int D, float scale, int causal,
    parallax_dtype_t in_dtype, void* workspace, size_t workspace_bytes,
    void* stream, const SavedFwd* saved) {
  if (B < 0 || N < 0 || H < 0)
    return fail(PARALLAX_ERR_INVALID_ARG, "negative size (B=%d N=%d H=%d)", B, N, H);
  parallax_status_t st = check_head_dim(D);
  if (st != PARALLAX_OK) return st;
  if (!valid_dtype(in_dtype)) return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  if (in_dtype != PARALLAX_BF16)
    return fail(PARALLAX_ERR_UNSUPPORTED, "parallax_bwd supports bf16 inputs only");
  if (!isfinite(scale)) return fail(PARALLAX_ERR_INVALID_ARG, "scale is not finite");
  if (B == 0 || N == 0 || H == 0) return ok();
  const int es = 2;
  const int64_t qs[3] = {q_sb, q_sn, q_sh}, ks[3] = {k_sb, k_sn, k_sh};
  const int64_t vs[3] = {v_sb, v_sn, v_sh}, rs[3] = {r_sb, r_sn, r_sh};
  const int64_t gs[3] = {g_sb, g_sn, g_sh};
  if ((st = check_input("q", q, es, qs, 3)) != PARALLAX_OK) return st;
  if ((st = check_input("k", k, es, ks, 3)) != PARALLAX_OK) return st;
  if ((st = check_input("v", v, es, vs, 3)) != PARALLAX_OK) return st;
  if ((st = check_input("rho", rho, es, rs, 3)) != PARALLAX_OK) return st;
  if ((st = check_input("dout", dout, es, gs, 3)) != PARALLAX_OK) return st;
  const int64_t dqs[3] = {dq_sb, dq_sn, dq_sh}, dks[3] = {dk_sb, dk_sn, dk_sh};
  const int64_t dvs[3] = {dv_sb, dv_sn, dv_sh}, drs[3] = {dr_sb, dr_sn, dr_sh};
  if ((st = check_output(dq, 4, dqs, 3)) != PARALLAX_OK) return st;
  if ((st = check_output(dk, 4, dks, 3)) != PARALLAX_OK) return st;
  if ((st = check_output(dv, 4, dvs, 3)) != PARALLAX_OK) return st;
  if ((st = check_output(drho, 4, drs, 3)) != PARALLAX_OK) return st;
  if ((st = check_grid((N + 15) / 16, H, B)) != PARALLAX_OK) return st;
  {
    // tiles of every input are addressed with 32-bit buffer offsets
    int64_t sn = q_sn;
    for (int64_t x : {k_sn, v_sn, r_sn, g_sn}) sn = x > sn ? x : sn;
    const int64_t rows = N > 64 ? N : 64;
    if (sn * 2 * rows + 2 * D > 0x7fffffffLL)
      return fail(PARALLAX_ERR_UNSUPPORTED,
                  "bf16 backward: one (b, h) slice of an input spans more than 2 GiB");
  }
  const size_t need = bwd_workspace_bytes(B, N, H);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PARALLAX_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (!aligned(workspace, 16))
    return fail(PARALLAX_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  float* stats = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;

  parallax::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.rho = rho; p.dout = dout;
  p.q_sb = q_sb; p.q_sn = q_sn; p.q_sh = q_sh;
  p.k_sb = k_sb; p.k_sn = k_sn; p.k_sh = k_sh;
  p.v_sb = v_sb; p.v_sn = v_sn; p.v_sh = v_sh;
  p.r_sb = r_sb; p.r_sn = r_sn; p.r_sh = r_sh;
  p.g_sb = g_sb; p.g_sn = g_sn; p.g_sh = g_sh;
  p.dq = dq; p.dk = dk; p.dv = dv; p.drho = drho;
  p.dq_sb = dq_sb; p.dq_sn = dq_sn; p.dq_sh = dq_sh;
  p.dk_sb = dk_sb; p.dk_sn = dk_sn; p.dk_sh = dk_sh;
  p.dv_sb = dv_sb; p.dv_sn = dv_sn; p.dv_sh = dv_sh;
  p.dr_sb = dr_sb; p.dr_sn = dr_sn; p.dr_sh = dr_sh;
  p.B = B; p.N = N; p.H = H;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  p.stats = stats;
  p.stats_w = stats;
  if (saved != nullptr) {
    // the query-block kernel forms the statistics from the saved tensors
    p.saved_out = saved->out;
    p.so_sb = saved->o_sb; p.so_sn = saved->o_sn; p.so_sh = saved->o_sh;
    p.saved_out_bf16 = saved->out_bf16 ? 1 : 0;
    p.saved_vbar = saved->vbar;
    p.saved_lse_rbar = saved->lse_rbar;
  } else {
    e = parallax::launch_bwd_stats_bf16(p, D, s);
    if (e != hipSuccess) return from_hip(e, "parallax_bwd statistics launch");
  }
  e = parallax::launch_bwd_bf16(p, D, s);
  return from_hip(e, "parallax_bwd launch");
}

}  // namespace

extern "C" {

parallax_status_t parallax_bwd(
    const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
    int64_t k_sb, int64_t k_sn, int64_t k_sh, const void* v, int64_t v_sb,
    int64_t v_sn, int64_t v_sh, const void* rho, int64_t r_sb, int64_t r_sn,
    int64_t r_sh, const void* dout, int64_t g_sb, int64_t g_sn, int64_t g_sh,
    float* dq, int64_t dq_sb, int64_t dq_sn, int64_t dq_sh, float* dk,
    int64_t dk_sb, int64_t dk_sn, int64_t dk_sh, float* dv, int64_t dv_sb,
    int64_t dv_sn, int64_t dv_sh, float* drho, int64_t dr_sb, int64_t dr_sn,
    int64_t dr_sh, int B, int N, int H, int D, float scale, int causal,
    parallax_dtype_t in_dtype, void* workspace, size_t workspace_bytes,
    void* stream) {
  return bwd_impl(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, v, v_sb, v_sn, v_sh, rho, r_sb,
                  r_sn, r_sh, dout, g_sb, g_sn, g_sh, dq, dq_sb, dq_sn, dq_sh, dk, dk_sb,
                  dk_sn, dk_sh, dv, dv_sb, dv_sn, dv_sh, drho, dr_sb, dr_sn, dr_sh, B, N, H,
                  D, scale, causal, in_dtype, workspace, workspace_bytes, stream, nullptr);
}

parallax_status_t parallax_bwd_saved(
    const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
    int64_t k_sb, int64_t k_sn, int64_t k_sh, const void* v, int64_t v_sb,
    int64_t v_sn, int64_t v_sh, const void* rho, int64_t r_sb, int64_t r_sn,
    int64_t r_sh, const void* dout, int64_t g_sb, int64_t g_sn, int64_t g_sh,
    const void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
    parallax_dtype_t out_dtype, const float* vbar, const float* lse_rbar, float* dq,
    int64_t dq_sb, int64_t dq_sn, int64_t dq_sh, float* dk, int64_t dk_sb,
    int64_t dk_sn, int64_t dk_sh, float* dv, int64_t dv_sb, int64_t dv_sn,
    int64_t dv_sh, float* drho, int64_t dr_sb, int64_t dr_sn, int64_t dr_sh, int B,
    int N, int H, int D, float scale, int causal, parallax_dtype_t in_dtype,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(out_dtype)) return fail(PARALLAX_ERR_INVALID_ARG, "unknown dtype");
  if (B > 0 && N > 0 && H > 0) {
    if (out == nullptr || vbar == nullptr || lse_rbar == nullptr)
      return fail(PARALLAX_ERR_INVALID_ARG, "out, vbar or lse_rbar is NULL");
    // o and vbar are read with 16-byte loads
    const int64_t os[3] = {o_sb, o_sn, o_sh};
    parallax_status_t st = check_input("out", out, dtype_bytes(out_dtype), os, 3);
    if (st != PARALLAX_OK) return st;
    if (!aligned(vbar, 16) || !aligned(lse_rbar, 8))
      return fail(PARALLAX_ERR_UNSUPPORTED,
                  "vbar must be 16-byte and lse_rbar 8-byte aligned");
  }
  const SavedFwd sv{out, o_sb, o_sn, o_sh, out_dtype == PARALLAX_BF16, vbar, lse_rbar};
  return bwd_impl(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, v, v_sb, v_sn, v_sh, rho, r_sb,
                  r_sn, r_sh, dout, g_sb, g_sn, g_sh, dq, dq_sb, dq_sn, dq_sh, dk, dk_sb,
                  dk_sn, dk_sh, dv, dv_sb, dv_sn, dv_sh, drho, dr_sb, dr_sn, dr_sh, B, N, H,
                  D, scale, causal, in_dtype, workspace, workspace_bytes, stream, &sv);
}

}  // extern "C"
