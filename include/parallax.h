/*
 * parallax.h -- C ABI of libparallax, the MI355X (gfx950) Parallax attention
 * hot path.
 *
 * Parallax attention keeps softmax attention and subtracts a learned
 * covariance correction. For query i with probe rho_i (the output of a
 * learned projection W_R applied to the layer input, computed by the caller)
 * and visible keys J_i, the zubnet.ai news item on Parallax ("Parallax
 * mantiene softmax ... correccion de covarianza aprendida", second
 * paragraph) defines the output as softmax attention minus the key-value
 * covariance contracted with rho_i; with W_R = 0 (rho = 0) it is plain
 * softmax attention. In formulas (scale = softmax scale):
 *
 *   p_ij  = softmax_j( scale * q_i . k_j )               over j in J_i
 *   vbar  = sum_j p_ij v_j,   kbar = sum_j p_ij k_j
 *   o_i   = vbar - sum_j p_ij (v_j - vbar) ((k_j - kbar) . rho_i)
 *
 * The probe contracts the key side; rho . k is not scaled. The library
 * evaluates this in one streaming pass over K and V (both branches share the
 * same KV stream, as the same paragraph describes), through
 *   o_i = vbar (1 + rbar) - sum_j p_ij r_ij v_j,  r_ij = rho_i . k_j,
 *   rbar = sum_j p_ij r_ij,
 * accumulated with online softmax in fp32.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller. The
 *    library never allocates, frees or synchronises; calls only enqueue
 *    work on `stream` (a hipStream_t passed as void*, NULL = null stream)
 *    and return. Device-side faults surface at the caller's next sync.
 *  - Strides are in ELEMENTS. The innermost (head_dim) stride is 1. Every
 *    base pointer must be 16-byte aligned and every stride times the
 *    element size a multiple of 16 bytes; otherwise
 *    PARALLAX_ERR_UNSUPPORTED.
 *  - Supported: head_dim D in {64, 128}; in_dtype PARALLAX_F32 or
 *    PARALLAX_BF16 (q, k, v, rho share it); out_dtype PARALLAX_F32 or
 *    PARALLAX_BF16. Query and key/value head counts are equal (except in
 *    parallax_decode_gqa). B and H are at most 65535 and the launch grid
 *    (about B * H * ceil(N / 16) workgroups, or B * kv heads * splits for
 *    grouped-query decode) below 2^31; larger problems return
 *    PARALLAX_ERR_UNSUPPORTED.
 *  - Arguments are validated on the host before any HIP call. A bad
 *    argument returns PARALLAX_ERR_INVALID_ARG / _UNSUPPORTED /
 *    _WORKSPACE and launches nothing. A failed launch returns
 *    PARALLAX_ERR_HIP. parallax_last_error() gives a per-thread message
 *    for the most recent failure.
 *  - Empty problems (B, H or N equal to 0) return PARALLAX_OK and launch
 *    nothing. A sequence with no visible keys gets a zero output row.
 *  - Non-finite inputs are not checked; they propagate.
 */
#ifndef PARALLAX_H_
#define PARALLAX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PARALLAX_API __attribute__((visibility("default")))
#else
#define PARALLAX_API
#endif

typedef enum {
  PARALLAX_OK = 0,
  PARALLAX_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum  */
  PARALLAX_ERR_UNSUPPORTED = 2, /* D, dtype, stride or alignment not served */
  PARALLAX_ERR_WORKSPACE = 3,   /* workspace missing or too small          */
  PARALLAX_ERR_HIP = 4          /* the HIP runtime reported an error       */
} parallax_status_t;

typedef enum { PARALLAX_F32 = 0, PARALLAX_BF16 = 1 } parallax_dtype_t;

/* Static description of a status code; never NULL. */
PARALLAX_API const char *parallax_status_string(parallax_status_t status);

/* Message describing the last failure on the calling thread ("" if none). */
PARALLAX_API const char *parallax_last_error(void);

/*
 * Number of KV splits parallax_decode uses for these sizes. num_splits > 0
 * requests that count (clamped to [1, ceil(Lmax / 64)]); num_splits == 0
 * asks for the library's choice, a pure function of (B, H, D, Lmax): about
 * one workgroup per compute unit of an MI355X (256) over the B * H streams,
 * splits of at least 256 keys, contexts under 1024 keys unsplit. Host-only,
 * no HIP call.
 */
PARALLAX_API parallax_status_t parallax_decode_splits(int B, int H, int D,
                                                      int Lmax, int num_splits,
                                                      int *splits_out);

/*
 * Device workspace in bytes needed by parallax_decode for these sizes and
 * split request (0 when one split suffices). Host-only, no HIP call.
 * Layout (informative): per (b, h, split) one fp32 record
 *   [m, l, A_r, 0, A_v[D], A_rv[D]]  (m in base-2 logit units).
 */
PARALLAX_API parallax_status_t parallax_decode_workspace_size(
    int B, int H, int D, int Lmax, int num_splits, size_t *bytes);

/*
 * Decode: one new query per sequence against a KV cache.
 *
 * Defining passage: the zubnet.ai news item on Parallax, second paragraph:
 * the output is softmax attention minus the key-value covariance
 * contracted with the probe, both branches read the same KV stream, and
 * decoding still needs the KV cache. One query per sequence attends to the
 * cached positions; the kernel is this library's own gfx950 design (the
 * page's H200 kernel is not described beyond its comparison).
 *
 *   q      [B, H, D]        element (b,h,d) at q[b*q_sb + h*q_sh + d]
 *   rho    [B, H, D]        probe, element at rho[b*r_sb + h*r_sh + d], or
 *                           NULL: plain softmax attention, the output for
 *                           rho = 0, computed without the rho.k products
 *                           and the covariance sums (r_sb, r_sh ignored)
 *   k_cache, v_cache [B, H, Lmax, D]
 *                           element (b,h,l,d) at [b*kv_sb + h*kv_sh + l*kv_sl + d]
 *   seqlens  device int32[B] or NULL. Sequence b attends to cache positions
 *            [0, min(seqlens[b], Lmax)); NULL means Lmax for all. Values
 *            <= 0 give a zero row. Positions at or beyond the length are
 *            never read. The cache already holds the new token's key/value.
 *   out    [B, H, D] of out_dtype, element at out[b*o_sb + h*o_sh + d]
 *   scale  softmax scale applied to q . k (1/sqrt(D) is the usual value)
 *   num_splits  0 = library choice, else requested split count
 *   workspace   device buffer of at least
 *               parallax_decode_workspace_size(...) bytes (may be NULL when
 *               that size is 0). Its contents need not be initialised; it
 *               must not be shared by calls that may run concurrently.
 *
 * Keys are split into contiguous ranges; each range is streamed once by one
 * workgroup that computes both q.k and rho.k from one load of each key row
 * and both accumulations from one load of each value row. Partial states
 * are merged by rescale-and-add in a second kernel when splits > 1.
 */
PARALLAX_API parallax_status_t parallax_decode(
    const void *q, int64_t q_sb, int64_t q_sh,
    const void *rho, int64_t r_sb, int64_t r_sh,
    const void *k_cache, const void *v_cache,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sl,
    const int32_t *seqlens,
    void *out, int64_t o_sb, int64_t o_sh,
    int B, int H, int D, int Lmax, float scale,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype,
    int num_splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * parallax_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results (bit for bit, same kernels) without the
 * workspace. Split records go to a fixed 4 MiB device array inside the
 * library (static storage: every GPU the library runs on holds its own copy
 * until the process ends; its address is looked up once per device, on the
 * device of `stream`, at that device's first call). The call itself
 * allocates nothing.
 *   Limit: a call whose split records (parallax_decode_workspace_size for
 *   the same sizes and num_splits) exceed 4 MiB = 4194304 bytes returns
 *   PARALLAX_ERR_WORKSPACE and launches nothing; the library's own split
 *   choice stays far below it (about 256 (b, h, split) records of 1040
 *   bytes at D = 128). One split needs no scratch at all.
 *   Calls that may overlap on one GPU (several streams, several host
 *   threads) share that GPU's array and race; serialise them. Nothing in the
 *   array needs to start at zero: every record is written before it is read.
 */
PARALLAX_API parallax_status_t parallax_decode_noalloc(
    const void *q, int64_t q_sb, int64_t q_sh,
    const void *rho, int64_t r_sb, int64_t r_sh,
    const void *k_cache, const void *v_cache,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sl,
    const int32_t *seqlens,
    void *out, int64_t o_sb, int64_t o_sh,
    int B, int H, int D, int Lmax, float scale,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype,
    int num_splits, void *stream);

/*
 * Device workspace in bytes needed by parallax_fwd for these sizes: for
 * bf16 inputs B * H * ceil(N / 64) * 64 * D * 2 (V packed as fp16 key
 * tiles), for fp32 inputs 0. Host-only, no HIP call.
 */
PARALLAX_API parallax_status_t parallax_fwd_workspace_size(
    int B, int N, int H, int D, parallax_dtype_t in_dtype, size_t *bytes);

/*
 * Number of KV splits parallax_decode_gqa uses for these sizes; paged is
 * nonzero for a call with a block table. num_splits 0 = its own choice,
 * splits of at least 128 keys: a workgroup serves h kv heads of one
 * sequence (h = the largest of 8, 4, 2, 1 dividing Hkv) when the cache is
 * paged, h is at least 4 and B * (Hkv / h) * Lmax reaches 2^17, or the
 * cache is contiguous and B * (Hkv / h) reaches 256 * 8 / h, and the splits
 * then aim at eight waves per compute unit; otherwise a workgroup serves
 * one kv head and the splits aim at about one workgroup per compute unit
 * over the B * Hkv streams. Host-only.
 */
PARALLAX_API parallax_status_t parallax_decode_gqa_splits(int B, int Hq, int Hkv, int D,
                                                          int Lmax, int paged, int num_splits,
                                                          int *splits_out);

/*
 * Workspace bytes for parallax_decode_gqa (0 when one split suffices).
 * Splits are as parallax_decode_gqa_splits(B, Hq, Hkv, D, Lmax, paged,
 * num_splits) plans them; one record per (b, query head, split). Host-only,
 * no HIP call.
 */
PARALLAX_API parallax_status_t parallax_decode_gqa_workspace_size(
    int B, int Hq, int Hkv, int D, int Lmax, int paged, int num_splits, size_t *bytes);

/*
 * Decode with grouped query heads and an optional paged KV cache.
 * Query head hq reads key-value head hq / (Hq / Hkv); Hq / Hkv must be 1,
 * 2, 4 or 8. Each key-value stream is read once per (b, kv head, split) and
 * feeds all query heads of its group (softmax and covariance branch).
 *
 *   q, rho   [B, Hq, D] bf16, element (b,h,d) at X[b*X_sb + h*X_sh + d]
 *   block_table == NULL: contiguous cache [B, Hkv, Lmax, D], element
 *            (b,hk,l,d) at cache[b*kv_sb + hk*kv_sh + l*kv_sl + d]
 *   block_table != NULL: paged cache of num_pages pages of page_size
 *            tokens (page_size a positive multiple of 8), element
 *            (page,t,hk,d) at cache[page*kv_sb + t*kv_sl + hk*kv_sh + d];
 *            position l of sequence b is in page block_table[b*bt_sb +
 *            l / page_size] (device int32) at row l % page_size. seqlens is
 *            then required; Lmax bounds the lengths (split planning uses
 *            it). Keys whose page index lies outside [0, num_pages) are
 *            skipped (never read).
 *   seqlens  device int32[B] or NULL (contiguous only: Lmax for all)
 *   out      [B, Hq, D] of out_dtype
 *   other arguments as parallax_decode; workspace of
 *   parallax_decode_gqa_workspace_size(...) bytes when splits > 1.
 * bf16 inputs only. The arithmetic per query head is that of
 * parallax_decode (zubnet.ai news item on Parallax, second paragraph); the
 * pages do not discuss grouped heads or paged caches, which are the
 * serving layouts of a KV cache that decoding keeps.
 */
PARALLAX_API parallax_status_t parallax_decode_gqa(
    const void *q, int64_t q_sb, int64_t q_sh,
    const void *rho, int64_t r_sb, int64_t r_sh,
    const void *k_cache, const void *v_cache,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sl,
    const int32_t *block_table, int64_t bt_sb, int page_size, int num_pages,
    const int32_t *seqlens,
    void *out, int64_t o_sb, int64_t o_sh,
    int B, int Hq, int Hkv, int D, int Lmax, float scale,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype,
    int num_splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Prefill (training/forward) over whole sequences.
 *
 * Defining passage: the zubnet.ai news item on Parallax, second paragraph
 * (softmax attention minus the key-value covariance contracted with the
 * probe rho_i = W_R x_i, in one pass over the keys and values that both
 * branches share), applied to every query with the causal key set. The
 * pages describe no prefill kernel; this tiled matrix-core design is the
 * library's own.
 *
 *   q, k, v, rho  [B, N, H, D]; tensor X's element (b,n,h,d) is at
 *                 X[b*X_sb + n*X_sn + h*X_sh + d] with its own strides.
 *   out           [B, N, H, D] of out_dtype with strides o_sb, o_sn, o_sh.
 *   causal        nonzero: query n sees keys 0..n (diagonal included);
 *                 zero: every query sees all N keys.
 *
 * bf16 inputs run on the matrix cores: q.k and rho.k as bf16 products with
 * fp32 accumulation; the probability-side products (p v and p r v) take
 * fp16 operands (p in [0,1], p*r and v converted from bf16), fp32
 * accumulation. fp16 holds bf16 values exactly except magnitudes above
 * 65504 or below 2^-14 (rounded as fp16 subnormals); |rho . k| must stay
 * below 65504. fp32 inputs are computed in fp32 throughout.
 *
 *   workspace   device buffer of at least parallax_fwd_workspace_size(...)
 *               bytes, 16-byte aligned (may be NULL when that size is 0).
 *               For bf16 inputs the call first writes V there as fp16 key
 *               tiles, transposed and in the order the matrix-core kernel
 *               loads them, then runs the attention kernel; both kernels run
 *               on `stream`. Contents need not be initialised; it must not
 *               be shared by calls that may run concurrently.
 */
PARALLAX_API parallax_status_t parallax_fwd(
    const void *q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
    const void *k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
    const void *v, int64_t v_sb, int64_t v_sn, int64_t v_sh,
    const void *rho, int64_t r_sb, int64_t r_sn, int64_t r_sh,
    void *out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
    int B, int N, int H, int D, float scale, int causal,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Device workspace in bytes needed by parallax_bwd (and parallax_bwd_saved)
 * for these sizes (bf16 inputs): the per-query statistics, 16 B per
 * (b, h, n), rounded up to 256 bytes. Host-only, no HIP call.
 */
PARALLAX_API parallax_status_t parallax_bwd_workspace_size(
    int B, int N, int H, int D, parallax_dtype_t in_dtype, size_t *bytes);

/*
 * Backward of parallax_fwd: given dout = dL/d out, writes dq, dk, dv, drho
 * (the gradients of L with respect to q, k, v and rho) for the same
 * B, N, H, D, scale and causal flag.
 *
 *   q, k, v, rho, dout  [B, N, H, D] bf16 (in_dtype must be PARALLAX_BF16),
 *                       element (b,n,h,d) at X[b*X_sb + n*X_sn + h*X_sh + d]
 *   dq, dk, dv, drho    [B, N, H, D] fp32, each with its own strides;
 *                       overwritten (not accumulated into)
 *   workspace           device buffer of at least
 *                       parallax_bwd_workspace_size(...) bytes, 16-byte
 *                       aligned; contents need not be initialised; not to
 *                       be shared by calls that may run concurrently.
 *
 * The gradient follows from the forward by the chain rule: with
 * g_i = dout_i, a_ij = g_i.v_j, b_i = g_i.vbar_i and
 * D_i = g_i.o_i + rbar_i b_i,
 *   ds_ij = p_ij (a_ij (1 + rbar_i - r_ij) + b_i r_ij - D_i),
 *   dr_ij = p_ij (b_i - a_ij),
 *   dq_i = scale sum_j ds_ij k_j,  drho_i = sum_j dr_ij k_j,
 *   dk_j = sum_i (scale ds_ij q_i + dr_ij rho_i),
 *   dv_j = sum_i p_ij (1 + rbar_i - r_ij) g_i.
 * Kernels (all on `stream`): a statistics pass that stores per query
 * log2-sum-exp, rbar, b and D (from q.k, rho.k and dout.v alone, with
 * b = sum_j p_ij a_ij and g_i.o_i = b_i (1 + rbar_i) - sum_j p_ij r_ij a_ij);
 * a query-block kernel for dq, drho;
 * and a key-block kernel for dk, dv (the transposed operands are read from
 * row-major tiles in LDS). Products q.k, rho.k and dout.v are bf16 with fp32
 * accumulation;
 * ds, dr and p (1 + rbar - r) enter the second contractions as bf16.
 */
PARALLAX_API parallax_status_t parallax_bwd(
    const void *q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
    const void *k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
    const void *v, int64_t v_sb, int64_t v_sn, int64_t v_sh,
    const void *rho, int64_t r_sb, int64_t r_sn, int64_t r_sh,
    const void *dout, int64_t g_sb, int64_t g_sn, int64_t g_sh,
    float *dq, int64_t dq_sb, int64_t dq_sn, int64_t dq_sh,
    float *dk, int64_t dk_sb, int64_t dk_sn, int64_t dk_sh,
    float *dv, int64_t dv_sb, int64_t dv_sn, int64_t dv_sh,
    float *drho, int64_t dr_sb, int64_t dr_sn, int64_t dr_sh,
    int B, int N, int H, int D, float scale, int causal,
    parallax_dtype_t in_dtype, void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * Prefill over packed variable-length sequences (bf16 inputs only).
 *
 *   q, k, v, rho  [T, H, D] bf16: sequence b is rows [cu_seqlens[b],
 *                 cu_seqlens[b+1]) of every tensor; element (t,h,d) of X at
 *                 X[t*X_sn + h*X_sh + d]
 *   out           [T, H, D] of out_dtype, same row ranges; rows outside
 *                 every sequence are not written
 *   cu_seqlens    device int32[B + 1], non-decreasing, cu_seqlens[0] >= 0;
 *                 the caller guarantees every row it names exists. Lengths
 *                 above max_seqlen are cut to max_seqlen.
 *   max_seqlen    longest sequence (sizes the grid and the workspace)
 *   workspace     parallax_fwd_workspace_size(B, max_seqlen, H, D, BF16)
 *                 bytes, 16-byte aligned (fp16 V^T tiles per sequence)
 *
 * Each sequence is computed exactly as parallax_fwd computes one batch
 * entry (causal within the sequence when `causal` is set): the same
 * kernels, with sequence b's rows addressed from cu_seqlens[b]. Query
 * blocks past a sequence's end exit at once, so the cost follows the
 * actual lengths. Errors as for parallax_fwd; fp32 inputs return
 * UNSUPPORTED, a NULL cu_seqlens INVALID_ARG.
 */
PARALLAX_API parallax_status_t parallax_fwd_varlen(
    const void *q, int64_t q_sn, int64_t q_sh,
    const void *k, int64_t k_sn, int64_t k_sh,
    const void *v, int64_t v_sn, int64_t v_sh,
    const void *rho, int64_t r_sn, int64_t r_sh,
    void *out, int64_t o_sn, int64_t o_sh,
    const int32_t *cu_seqlens, int B, int max_seqlen, int H, int D,
    float scale, int causal, parallax_dtype_t in_dtype, parallax_dtype_t out_dtype,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training forward: parallax_fwd (bf16 inputs, same arguments and output)
 * that also keeps what the backward needs, so parallax_bwd_saved can skip
 * recomputing the forward:
 *   vbar      [B, N, H, D] fp32, contiguous: the softmax mean of the values
 *             sum_j p_ij v_j of every query (16-byte aligned)
 *   lse_rbar  [B, H, N] pairs of fp32, contiguous: {lse2, rbar} per query,
 *             lse2 = log2 sum_j 2^(scale q.k_j log2 e), rbar = sum_j p_ij
 *             rho.k_j (8-byte aligned)
 * Errors as parallax_fwd; UNSUPPORTED for fp32 inputs.
 */
PARALLAX_API parallax_status_t parallax_fwd_train(
    const void *q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
    const void *k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
    const void *v, int64_t v_sb, int64_t v_sn, int64_t v_sh,
    const void *rho, int64_t r_sb, int64_t r_sn, int64_t r_sh,
    void *out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
    float *vbar, float *lse_rbar,
    int B, int N, int H, int D, float scale, int causal,
    parallax_dtype_t in_dtype, parallax_dtype_t out_dtype,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward from a training forward's saved tensors: the gradients of
 * parallax_bwd (same arguments, workspace and results up to rounding order)
 * with the per-query statistics taken from the forward's output `out`
 * (fp32 or bf16, its own strides), vbar and lse_rbar (as written by
 * parallax_fwd_train with the same q, k, v, rho, scale and causal flag)
 * instead of a second forward pass: b_i = dout_i . vbar_i and
 * D_i = dout_i . o_i + rbar_i b_i are formed by the query-block gradient
 * kernel as it starts (two launches per call). A bf16 `out` rounds D_i;
 * fp32 keeps the parallax_bwd precision. `out` must be 16-byte aligned with
 * strides whose byte size is a multiple of 16, vbar 16-byte aligned
 * (otherwise PARALLAX_ERR_UNSUPPORTED).
 */
PARALLAX_API parallax_status_t parallax_bwd_saved(
    const void *q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
    const void *k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
    const void *v, int64_t v_sb, int64_t v_sn, int64_t v_sh,
    const void *rho, int64_t r_sb, int64_t r_sn, int64_t r_sh,
    const void *dout, int64_t g_sb, int64_t g_sn, int64_t g_sh,
    const void *out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
    parallax_dtype_t out_dtype, const float *vbar, const float *lse_rbar,
    float *dq, int64_t dq_sb, int64_t dq_sn, int64_t dq_sh,
    float *dk, int64_t dk_sb, int64_t dk_sn, int64_t dk_sh,
    float *dv, int64_t dv_sb, int64_t dv_sn, int64_t dv_sh,
    float *drho, int64_t dr_sb, int64_t dr_sn, int64_t dr_sh,
    int B, int N, int H, int D, float scale, int causal,
    parallax_dtype_t in_dtype, void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * Defining passage: the zubnet.ai news item on Parallax, second paragraph
 * (the probe rho_i = W_R x_i, W_R a learnable projection of the layer
 * input), and the encorp.ai blog "Integraciones de IA personalizadas tras
 * la atencion Parallax", section "Parallax conserva softmax..." (W_R = 0 is
 * exactly softmax attention, so an existing layer converts with zeros).
 *
 * Fused input projection of a Parallax layer: y = x W^T in bf16 with fp32
 * accumulation, rounded to bf16 (nearest even). With W the output features
 * of the q, k, v and probe projections stacked ([W_Q; W_K; W_V; W_R]), one
 * call yields q, k, v and rho = W_R x side by side in each row of y; viewed
 * as [M, H, D] with strides (y_st, D), each part is a valid input of
 * parallax_fwd, parallax_fwd_varlen or, per token, the decode entry points.
 * W_R = 0 rows give rho = 0, i.e. plain softmax attention.
 *
 *   x  [M, K] bf16, element (m, k) at x[m*x_st + k]      (layer input)
 *   w  [N, K] bf16, element (n, k) at w[n*w_st + k]      (stacked weights)
 *   y  [M, N] bf16, element (m, n) at y[m*y_st + n]
 *   N a multiple of 256, K a positive multiple of 64, M any (>= 0).
 *   Pointers 16-byte aligned, row strides multiples of 8 elements and at
 *   least the row length.
 * Errors: INVALID_ARG for NULL pointers, negative sizes or short strides;
 * UNSUPPORTED for other dtypes, N or K off the multiples, misalignment.
 * Enqueued on `stream`; allocates nothing.
 */
PARALLAX_API parallax_status_t parallax_project(const void *x, int64_t x_st,
                                                const void *w, int64_t w_st,
                                                void *y, int64_t y_st,
                                                int M, int N, int K,
                                                parallax_dtype_t dtype, void *stream);

/*
 * Measurement reference, not part of the attention path: reads `bytes`
 * bytes at `src` with the 16-byte streaming loads of the decode kernels and
 * XORs every 32-bit word into *sink (device uint32; the caller sets its
 * initial value; one atomic XOR per wave). Its duration gives the plain
 * HBM read rate against which the decode kernels' bandwidth is read.
 *   src    device pointer, 16-byte aligned; bytes >= 0, a multiple of 16.
 *   sink   device pointer, 4-byte aligned, not NULL.
 * Errors: INVALID_ARG for NULL pointers or a negative size, UNSUPPORTED
 * for misalignment or a size not a multiple of 16. Enqueued on `stream`.
 */
PARALLAX_API parallax_status_t parallax_stream_read(const void *src, int64_t bytes,
                                                    uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_H_ */
