/*
 * attn.h - C ABI of the MI355X (gfx950) fused softmax-attention forward library.
 *
 * What the library computes, for every query row of every head: the softmax
 * attention o = softmax(scale * q K^T) V over the keys the row may see, and
 * its base-2 log-sum-exp lse2 = log2(sum_j exp(scale * <q, k_j>))
 * ("Flywheel Attention: Attention Kernels Built for the TPU", section 1;
 * "Writing Page Attention with PyPTO", section 1.1; "TokenSpeed-MLA",
 * kernel capability summary and packed-query paragraph for base-2 LSE).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     keeps none of them after the call returns. Scalars are host values.
 *   - Work is enqueued on the caller's HIP stream; no call synchronises,
 *     allocates or frees memory, or reads device memory on the host, so the
 *     calls may be captured in a HIP graph. The caller keeps every buffer
 *     alive until the stream has executed the work.
 *   - Every entry point returns attn_status_t and never aborts, throws or
 *     prints. Arguments are validated on the host before anything is
 *     enqueued; on an error nothing is enqueued and attn_last_error() holds
 *     a one-line reason (thread-local, valid until the next call on that
 *     thread).
 *   - Device-array CONTENTS are preconditions, not checked: block_table
 *     entries a request uses must lie in [0, num_pages); seq_lens and
 *     cu_seqlens must respect the max_* bounds passed alongside. Violating
 *     them is undefined behaviour (the kernel would read another request's
 *     pages: "Writing Page Attention with PyPTO", section 5.2 callout).
 *   - Table entries past a request's last page, and the slots of its last
 *     page past its length, are never read ("Writing Page Attention with
 *     PyPTO", section 9: the tail has two boundaries); their contents,
 *     NaN included, cannot change the output.
 *   - Query head h reads KV head h / (num_q_heads / num_kv_heads)
 *     ("Writing Page Attention with PyPTO", sections 1.2-1.3).
 *   - A causal row is aligned bottom-right: with Lq query rows and Lk keys,
 *     row i sees keys j <= Lk - Lq + i ("TokenSpeed-MLA", prefill command
 *     with bottom-right alignment, and the window_left row bound).
 *   - A row that sees no key gets o = 0 and lse = -inf ("TokenSpeed-MLA",
 *     section "SM107 decode").
 *   - Strides are in ELEMENTS of the stored type. The last dimension of
 *     every tensor is contiguous, and every row start is 16-byte aligned.
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,          /* null pointer, bad size, inconsistent shapes  */
  ATTN_ERR_UNSUPPORTED = 2,          /* valid request the library has no kernel for    */
  ATTN_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < attn_decode_workspace_size() */
  ATTN_ERR_HIP = 4                   /* a kernel launch failed                         */
} attn_status_t;

typedef enum {
  ATTN_BF16 = 0,       /* bfloat16                                                  */
  ATTN_FP8_E4M3 = 1,   /* OCP FP8 E4M3 ("fn": no infinities), one scale per tensor  */
  ATTN_FP32 = 2
} attn_dtype_t;

/* ------------------------------------------------------------------------
 * Ragged prefill over dense or paged KV ("TokenSpeed-MLA", kernel capability
 * summary, MLA Prefill: Q [sum q_lens, h_q, d_qk], K [sum kv_lens, h_k, d_qk],
 * V [sum kv_lens, h_k, d_v]; the query and key packings may differ).
 *
 *   q      bf16 [total_q, Hq, Dqk], strides q_stride_tok / q_stride_head.
 *   k, v   dense mode (block_table == NULL): bf16 [total_kv, Hkv, D], request
 *          b owns rows cu_seqlens_kv[b] .. cu_seqlens_kv[b+1]-1; the *_page
 *          strides are ignored.
 *          paged mode (block_table != NULL): bf16 [num_pages, page_size, Hkv,
 *          D]; token j of request b is slot j % page_size of page
 *          block_table[b * block_table_stride + j / page_size]; request b has
 *          seq_lens_kv[b] keys ("Writing Page Attention with PyPTO", sections
 *          1.2 and 5.2).
 *   cu_seqlens_q   int32 [batch + 1], request b owns query rows
 *                  cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1.
 *   max_seqlen_q, max_seqlen_kv   host upper bounds of the per-request lengths.
 *                  With max_seqlen_kv == 0 no row sees a key (O = 0, LSE =
 *                  -inf) and k, v (and, paged, the pages) may be empty/NULL;
 *                  with max_seqlen_q == 0 the call does nothing.
 *   causal         0 or 1 (bottom-right aligned).
 *   o      bf16 [total_q, Hq, Dv], strides o_stride_tok / o_stride_head.
 *   lse    optional float32 [total_q, Hq] contiguous, base 2; NULL to skip.
 *   window_enabled, window_left   sliding window ("TokenSpeed-MLA", kernel
 *          capability summary, window_left): with window_enabled = 1, query
 *          row i of a request with Lq queries and Lk keys also skips keys
 *          j < Lk - Lq - window_left + i (window_left >= 0 keys of context
 *          before the query block); window_enabled = 0 (a zeroed struct)
 *          is the full history.
 *   total_q, kv_splits, workspace   key splits (bf16 only): with a
 *          workspace of attn_prefill_workspace_size(p) bytes (16-byte
 *          aligned) and total_q set, the keys of each query tile may be
 *          walked by several workgroups whose partials are merged by log-sum-
 *          exp. With kv_splits = 0 (the planner chooses) a missing or too
 *          small workspace, or an o that is not contiguous, runs the call
 *          unsplit. A forced kv_splits > 1 is an error instead: FP8 inputs
 *          or a non-contiguous o give ATTN_ERR_UNSUPPORTED, total_q <= 0
 *          ATTN_ERR_INVALID_ARG, a missing or too small workspace
 *          ATTN_ERR_WORKSPACE_TOO_SMALL and a misaligned one
 *          ATTN_ERR_INVALID_ARG (the split count is capped at one split per
 *          64 keys of max_seqlen_kv, so a forced count may shrink to one, which
 *          needs no workspace). Results equal the unsplit ones up to
 *          rounding. total_q must equal cu_seqlens_q[batch]: query rows at
 *          or past a smaller total_q are not written (nor is the workspace
 *          beyond its size); with a larger one, the rows of o (and lse)
 *          past cu_seqlens_q[batch] receive unspecified values.
 *   qkv_dtype  ATTN_BF16 (a zeroed struct; the scales are ignored), or
 *          ATTN_FP8_E4M3: q, k and v hold E4M3 codes with per-tensor
 *          dequantisation scales q_scale, k_scale, v_scale > 0 (value = code
 *          * scale), the MLA-shaped FP8 prefill of "TokenSpeed-MLA" (prefill
 *          command: FP8 E4M3 inputs, q and k 192 wide; kernel capability
 *          summary: V d_v wide, output BF16, LSE FP32). Strides count
 *          elements of one byte.
 * Supported: bf16: Dqk == Dv in {64, 128, 256}, dense or paged; FP8: dense
 * mode with Dqk = 192 and Dv = 128. Hq % Hkv == 0; page_size a power of two
 * >= 16 (paged mode).
 * ---------------------------------------------------------------------- */
typedef struct {
  const void *q;
  int64_t q_stride_tok, q_stride_head;
  const void *k, *v;
  int64_t k_stride_page, k_stride_tok, k_stride_head;
  int64_t v_stride_page, v_stride_tok, v_stride_head;
  const int32_t *cu_seqlens_q;
  const int32_t *cu_seqlens_kv;      /* dense mode only */
  const int32_t *seq_lens_kv;        /* paged mode only */
  const int32_t *block_table;        /* NULL selects dense mode */
  int32_t block_table_stride;        /* elements between consecutive rows of block_table */
  int32_t page_size;
  int32_t num_pages;
  int32_t batch, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v;
  int32_t max_seqlen_q, max_seqlen_kv;
  float softmax_scale;
  int32_t causal;
  void *o;
  int64_t o_stride_tok, o_stride_head;
  float *lse;
  int32_t window_enabled;            /* 0: full history */
  int32_t window_left;               /* keys of context when window_enabled */
  attn_dtype_t qkv_dtype;            /* ATTN_BF16 (0) or ATTN_FP8_E4M3 */
  float q_scale, k_scale, v_scale;   /* FP8 dequantisation scales */
  int32_t total_q;                   /* query rows of q (sum of q_lens); needed for key splits */
  int32_t kv_splits;                 /* 0: the planner chooses; 1: no split; > 1: forced */
  void *workspace;                   /* key-split partials; NULL runs without splits */
  size_t workspace_bytes;
} attn_prefill_params;

/* Workspace bytes attn_prefill will use for p: S * total_q * Hq * (Dv + 1) * 4
 * when the plan splits the keys of each query tile into S > 1 ranges (bf16,
 * contiguous o [total_q, Hq, Dv], total_q > 0), else 0. With kv_splits = 0
 * the planner splits when the workgroups of the query tiles (counted from
 * total_q) fill at most half of the CUs' slots (toward one full round; the
 * CU count is the current device's, or 256 when no device is visible) or
 * leave a last round at most three quarters full (four splits), with no
 * split under 8192 keys (long keys, few query rows); each split's
 * normalised partial and LSE are then merged by attn_merge_lse's reducer.
 * Only shapes and scalars are examined. */
size_t attn_prefill_workspace_size(const attn_prefill_params *p);

/* Enqueue ragged prefill. Returns ATTN_OK, ATTN_ERR_INVALID_ARG,
 * ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE_TOO_SMALL (forced key splits
 * only) or ATTN_ERR_HIP. */
attn_status_t attn_prefill(const attn_prefill_params *p, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Paged decode with split-KV partials merged by log-sum-exp ("TokenSpeed-MLA",
 * sections "Decode performance" and "Key Optimization ... Group q_seqlen and
 * num_heads into BMM1 M"; "Writing Page Attention with PyPTO", sections 1-9).
 *
 *   q          [batch, q_len, Hq, Dqk] contiguous, in q_dtype: bf16 (0, a
 *              zeroed struct), or ATTN_FP8_E4M3 codes with the per-tensor
 *              dequantisation scale q_scale (value = code * q_scale), for an
 *              MLA-shaped FP8 cache only: the FP8 decode path whose query and
 *              latent cache are both FP8 ("TokenSpeed-MLA", MLA Decode in the
 *              kernel capability summary); its QK product runs on the FP8
 *              matrix instruction. q_scale is ignored for bf16 q.
 *   k_cache    [num_pages, page_size, Hkv, Dqk] in kv_dtype, strides k_stride_*.
 *   v_cache    [num_pages, page_size, Hkv, >= Dv] in kv_dtype, strides
 *              v_stride_*; V is the first Dv entries of each row. For an
 *              MLA-shaped latent cache pass the same pointer and strides as
 *              k_cache with Hkv = 1, Dqk = 576, Dv = 512: K is the whole row
 *              and V its first 512 entries, read once for both.
 *   kv_dtype   ATTN_BF16, or ATTN_FP8_E4M3 with per-tensor dequantisation
 *              scales k_scale / v_scale (value = code * scale); must be 1.0
 *              for bf16. An MLA-shaped FP8 cache needs k_scale == v_scale.
 *   seq_lens   int32 [batch]: keys of each request (0 allowed).
 *   block_table int32, row b at block_table + b * block_table_stride.
 *   max_seq_len host upper bound of seq_lens; plans the split count. With
 *              max_seq_len == 0 no row sees a key (O = 0, LSE = -inf) and the
 *              caches and block_table may be empty/NULL (num_pages 0).
 *   q_len      1..4 query tokens per request; row (t, h) of a causal request
 *              sees keys j <= seq_len - q_len + t.
 *   num_splits 0 lets the planner choose; otherwise the number of KV splits
 *              of every request. The GQA planner's choice (batch <= 512) is
 *              key ranges: the 32-key tiles of all requests, in request
 *              order, cut into K ranges of equal length (K = two waves per
 *              SIMD of the current device / (Hkv * q_groups), at most 512), so
 *              every wave walks the same number of keys ("Writing Page
 *              Attention with PyPTO", section 1.3: equal tasks keep every core
 *              busy to the end); a request inside one range is written
 *              directly, the pieces of the others are merged by LSE.
 *   workspace  device scratch of at least attn_decode_workspace_size(p)
 *              bytes (may be NULL when that is 0); contents undefined after.
 *   o          bf16 [batch, q_len, Hq, Dv] contiguous.
 *   lse        optional float32 [batch, q_len, Hq], base 2; NULL to skip.
 *   window_enabled, window_left   sliding window: with window_enabled = 1,
 *              row (t, h) also skips keys j < seq_len - q_len - window_left
 *              + t ("TokenSpeed-MLA", kernel capability summary,
 *              window_left); the walk starts at the window, so its cost
 *              tracks the window. 0 (a zeroed struct): full history.
 *   packed_q   0: the G query heads and F folded query tokens form the MFMA
 *              rows of a unit; 1: rows are packed continuously as
 *              t * G + g over the q_len tokens ("TokenSpeed-MLA", packed-
 *              query paragraph), so H96 with q_len 4 needs 3 tiles of 128
 *              rows instead of 4; the last tile may be partial. Output and
 *              LSE layouts are unchanged.
 *   total_kv_tokens   optional host-side sum of seq_lens (0: unknown). With
 *              num_splits = 0 it caps the key ranges at one per 8 tiles of
 *              the batch (small batches); for GQA batches above 512 it sizes
 *              per-request splits so that every unit is resident at once
 *              (units <= (total / S_len + batch) * Hkv * q_groups fit one
 *              round of the waves the current device's CUs hold). It only
 *              changes the plan, never the result.
 * Supported: (Dqk, Dv) in {(64,64), (128,128), (256,256)} with bf16 KV and
 * (576, 512) with Hkv == 1 and bf16 or FP8 KV; Hq % Hkv == 0; page_size a
 * power of two >= 16.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void *q;
  const void *k_cache, *v_cache;
  int64_t k_stride_page, k_stride_tok, k_stride_head;
  int64_t v_stride_page, v_stride_tok, v_stride_head;
  attn_dtype_t kv_dtype;
  float k_scale, v_scale;
  const int32_t *seq_lens;
  const int32_t *block_table;
  int32_t block_table_stride;
  int32_t batch, q_len, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v;
  int32_t page_size, num_pages, max_seq_len;
  float softmax_scale;
  int32_t causal;
  int32_t num_splits;
  void *workspace;
  size_t workspace_bytes;
  void *o;
  float *lse;
  int32_t window_enabled;   /* 0: full history */
  int32_t window_left;      /* keys of context when window_enabled */
  int32_t packed_q;         /* 0: folded rows; 1: continuous token * G + head rows */
  int64_t total_kv_tokens;  /* planner hint: host sum of seq_lens, 0 = unknown */
  attn_dtype_t q_dtype;     /* ATTN_BF16 (0) or ATTN_FP8_E4M3 (MLA-shaped FP8 cache only) */
  float q_scale;            /* fp8 q: value = code * q_scale */
} attn_decode_params;

/* How attn_decode_paged will decompose a call (host-only; no device access). */
typedef struct {
  int32_t group;          /* G = Hq / Hkv: query heads per KV head                     */
  int32_t fold;           /* F: query tokens folded with the G heads into MFMA rows
                             (1 with packed_q)                                          */
  int32_t q_groups;       /* row blocks per (request, KV head): q_len / F, or
                             ceil(G * q_len / rows_per_unit) with packed_q              */
  int32_t rows_per_unit;  /* rows computed together: G * F, or the MFMA tile rows (128
                             for the latent shape, 16 otherwise) capped at G * q_len
                             with packed_q                                             */
  int32_t num_splits;     /* S: KV splits per (request, KV head, q-group); 0 with key
                             ranges                                                     */
  int32_t split_tokens;   /* keys per split (the last one of a request may be shorter);
                             0 with key ranges                                          */
  int64_t num_units;      /* workgroups of the split kernel                             */
  size_t workspace_bytes; /* splits: S * R * (Dv + 1) * 4 with R = batch * q_len * Hq,
                             0 if S == 1; key ranges: (K + batch) * q_len * Hq * (Dv + 1)
                             * 4, 0 if K == 1                                           */
  int32_t key_ranges;     /* K > 0: the GQA plan that cuts the 32-key tiles of all
                             requests, in request order, into K ranges of (almost) equal
                             length, one per Hkv * q_groups waves; 0: per-request splits */
} attn_decode_plan_info;

/* Fill *info with the plan for p. Only shapes and scalars are examined (data
 * pointers may be NULL). ATTN_OK, ATTN_ERR_INVALID_ARG or ATTN_ERR_UNSUPPORTED. */
attn_status_t attn_decode_plan(const attn_decode_params *p, attn_decode_plan_info *info);

/* Workspace bytes attn_decode_paged needs for p (0 when one split suffices or
 * the shapes are invalid). Only shapes and scalars are examined. */
size_t attn_decode_workspace_size(const attn_decode_params *p);

/* Enqueue the split kernel and, when the plan has partials (workspace_bytes
 * > 0), the merge. Returns ATTN_OK, ATTN_ERR_INVALID_ARG,
 * ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE_TOO_SMALL or ATTN_ERR_HIP. */
attn_status_t attn_decode_paged(const attn_decode_params *p, hipStream_t stream);

/* The two kernels of attn_decode_paged, enqueued separately ("TokenSpeed-
 * MLA", section "Decode performance": the split-KV kernel, then a second
 * kernel that reduces its partials), for callers that schedule other work
 * between them or time them apart. attn_decode_paged_split writes the rows
 * the plan finishes in one unit to o / lse and the partials of the others
 * to the workspace; attn_decode_paged_merge, enqueued after it with the
 * same parameters and workspace contents, writes the remaining rows (and
 * does nothing when the plan has no partials). Together they give
 * attn_decode_paged's result bit for bit. Same arguments, validation and
 * return codes as attn_decode_paged. */
attn_status_t attn_decode_paged_split(const attn_decode_params *p, hipStream_t stream);
attn_status_t attn_decode_paged_merge(const attn_decode_params *p, hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): attn_decode_paged with
 * the split partials in a scratch array the library holds on each device
 * (128 MiB, kept until the process ends) instead of a caller workspace;
 * p->workspace and p->workspace_bytes are ignored. It allocates nothing. A
 * plan whose partials exceed the scratch (attn_decode_workspace_size(p) >
 * 128 MiB) returns ATTN_ERR_WORKSPACE_TOO_SMALL before anything is enqueued;
 * pass num_splits to plan fewer splits. Every call on one device shares its
 * scratch: calls that overlap on one device (other streams, other threads)
 * race and must be ordered by the caller. Results equal attn_decode_paged's
 * bit for bit (the same plan and kernels). Returns as attn_decode_paged, or
 * ATTN_ERR_HIP when the scratch's device address cannot be obtained. */
attn_status_t attn_decode_paged_noalloc(const attn_decode_params *p, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Merge split partials by log-sum-exp ("TokenSpeed-MLA", section "Decode
 * performance": a second kernel reduces the split-KV partial results; section
 * "FP8 split-KV partial storage": partials and log-sum-exp in FP32).
 *
 *   o_parts    float32 [num_splits, num_rows, head_dim_v]: per split, the
 *              output normalised over that split's keys.
 *   lse_parts  float32 [num_splits, num_rows]: base-2 log-sum-exp of each
 *              split's scores; -inf marks a split with no key (its o_parts
 *              row is then not read).
 *   o          [num_rows, head_dim_v] in o_dtype (ATTN_BF16 or ATTN_FP32):
 *              sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M), M = max_i lse_i.
 *   lse_out    optional float32 [num_rows]: M + log2(sum_i 2^(lse_i - M)).
 * A row whose splits are all -inf gets o = 0 and lse = -inf.
 * Supported: 1 <= num_splits <= 256; head_dim_v a multiple of 4, <= 1024.
 * ---------------------------------------------------------------------- */
attn_status_t attn_merge_lse(const float *o_parts, const float *lse_parts,
                             int32_t num_splits, int64_t num_rows, int32_t head_dim_v,
                             void *o, attn_dtype_t o_dtype, float *lse_out,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * K/V cache append: the step before a decode reads the cache ("Writing Page
 * Attention with PyPTO", section 4.2: the current token's K and V go to the
 * cache slot slot_mapping names; section 4.3: the slot is clamped at zero
 * BEFORE the layer base is added, so a warm-up slot of -1 writes row 0 of
 * the layer and never the last row of the previous layer; section 9.2: the
 * layer base selects one layer of a packed multi-layer cache).
 *
 *   k_new      bf16 [num_tokens, Hkv, Dk], strides k_new_stride_tok /
 *              k_new_stride_head.
 *   v_new      bf16 [num_tokens, Hkv, Dv], strides v_new_stride_*; NULL
 *              when the cache has no separate V (a latent cache, whose V is
 *              the first Dv entries of each K row).
 *   k_cache, v_cache   paged caches in cache_dtype viewed as token rows: row r
 *              is slot r % page_size of page r / page_size, at
 *              page * *_stride_page + slot * *_stride_tok + head *
 *              *_stride_head. v_cache is ignored when v_new is NULL.
 *   cache_dtype ATTN_BF16 (the bits are copied) or ATTN_FP8_E4M3: code =
 *              the E4M3 value nearest to x / scale (binary32 quotient,
 *              ties to even, |x / scale| > 448 saturating to +-448), with
 *              k_scale / v_scale > 0; the scales must be 1.0 for bf16.
 *   slot_mapping int64 [num_tokens] (device): row of token i within the
 *              layer; a negative entry is taken as 0.
 *   layer_base_rows   first token row of the layer (>= 0).
 *   num_cache_rows    token rows the cache holds (pages * page_size); a
 *              token whose row layer_base_rows + max(slot, 0) is at or past
 *              it is not written (a bound check, not an error: device
 *              contents are never read on the host).
 * Tokens that address the same row race: each 8-element piece of the row
 * ends up holding the same piece of one of them. NaN inputs give an
 * unspecified code in FP8 caches.
 * Supported: Dk, Dv multiples of 8 and <= 1024; page_size a power of two;
 * 16-byte aligned rows (8-byte aligned for FP8 caches).
 * ---------------------------------------------------------------------- */
typedef struct {
  const void *k_new;
  int64_t k_new_stride_tok, k_new_stride_head;
  const void *v_new;
  int64_t v_new_stride_tok, v_new_stride_head;
  void *k_cache;
  int64_t k_stride_page, k_stride_tok, k_stride_head;
  void *v_cache;
  int64_t v_stride_page, v_stride_tok, v_stride_head;
  attn_dtype_t cache_dtype;
  float k_scale, v_scale;
  const int64_t *slot_mapping;
  int64_t layer_base_rows;
  int64_t num_cache_rows;
  int32_t num_tokens, num_kv_heads, head_dim_k, head_dim_v;
  int32_t page_size;
} attn_cache_append_params;

/* Enqueue the append. ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED or
 * ATTN_ERR_HIP. num_tokens == 0 enqueues nothing. */
attn_status_t attn_cache_append(const attn_cache_append_params *p, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MLA K/V pack + FP8 quantise ("TokenSpeed-MLA", kernel capability summary:
 * one fused kernel in place of concatenate + cast + cast in chunked prefill,
 * strided inputs and caller-provided outputs).
 *
 *   k_nope     bf16 [num_tokens, H, d_nope], strides k_nope_stride_tok/_head.
 *   k_rope     bf16 [num_tokens, d_rope], stride k_rope_stride_tok: one
 *              vector per token, shared by every head.
 *   v          bf16 [num_tokens, H, d_v], strides v_stride_tok/_head.
 *   k_out      E4M3 codes [num_tokens, H, d_nope + d_rope]: per head the
 *              d_nope entries of k_nope, then the token's d_rope entries.
 *   v_out      E4M3 codes [num_tokens, H, d_v].
 *   k_scale, v_scale  per-tensor scales (> 0): code = E4M3(x / scale) with
 *              the rounding and saturation of attn_cache_append (NaN
 *              inputs give an unspecified code).
 * Supported: d_nope, d_rope, d_v multiples of 8; 16-byte aligned input rows
 * and 8-byte aligned output rows; per-head strides below 2^24 elements.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void *k_nope;
  int64_t k_nope_stride_tok, k_nope_stride_head;
  const void *k_rope;
  int64_t k_rope_stride_tok;
  const void *v;
  int64_t v_stride_tok, v_stride_head;
  void *k_out;
  int64_t k_out_stride_tok, k_out_stride_head;
  void *v_out;
  int64_t v_out_stride_tok, v_out_stride_head;
  float k_scale, v_scale;
  int32_t num_tokens, num_heads, d_nope, d_rope, d_v;
} attn_mla_kv_pack_params;

/* Enqueue the pack. ATTN_OK, ATTN_ERR_INVALID_ARG or ATTN_ERR_HIP.
 * num_tokens == 0 enqueues nothing. */
attn_status_t attn_mla_kv_pack_fp8(const attn_mla_kv_pack_params *p, hipStream_t stream);

/* Static name of a status code. */
const char *attn_status_string(attn_status_t s);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */
