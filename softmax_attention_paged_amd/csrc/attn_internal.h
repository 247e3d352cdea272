// Internal interface between the C-ABI layer (host validation and planning)
// and the kernel launchers. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/attn.h"

namespace attn {

// Everything the GQA split-decode kernel needs, already validated.
struct DecodeGqaArgs {
  const void *q;                 // bf16 [B, q_len, Hq, D]
  const void *k_cache, *v_cache;
  int64_t k_stride_page, k_stride_tok, k_stride_head;
  int64_t v_stride_page, v_stride_tok, v_stride_head;
  const int32_t *seq_lens;
  const int32_t *block_table;
  int32_t block_table_stride;
  int32_t batch, q_len, num_q_heads, num_kv_heads, head_dim;
  int32_t page_shift;            // log2(page_size)
  int32_t group, fold, q_groups, rows;
  int32_t packed;                // rows numbered t * group + g across the q_len tokens
  int32_t num_splits, split_tokens;
  // > 0: even key ranges instead of per-request splits. The tiles of all
  // requests, in request order, are cut into min(key_ranges, tiles) ranges
  // of (almost) equal length, one per group of Hkv * q_groups waves; a
  // request's piece in range g has partial slot g + b.
  int32_t key_ranges;
  float scale_log2;              // softmax_scale * log2(e)
  int32_t causal;
  int32_t window_left;           // keys of context before the query block; -1: full history
  // outputs: final (one split, or a request inside one key range) or partials
  void *o;                       // bf16 [B, q_len, Hq, D]
  float *lse;                    // optional [B, q_len, Hq]
  float *o_parts;                // splits: [S, R, D]; key ranges: [key_ranges + B, q_len * Hq, D]
  float *lse_parts;              // splits: [S, R]; key ranges: [key_ranges + B, q_len * Hq]
};

// Key ranges of the GQA decode (gqa_request_tiles in device_common.h counts
// a request's tiles).
constexpr int kMaxKeyRanges = 512;      // pieces one row may be merged from
constexpr int kKeyRangeMaxBatch = 512;  // requests the kernels scan (8 per lane)

// MLA-shaped decode: one latent KV head, K = the 576-wide row, V its first 512.
struct DecodeMlaArgs {
  const void *q;                 // bf16 [B, q_len, H, 576]
  const void *kv_cache;          // bf16 or fp8 codes [pages, ps, 1, 576]
  int64_t kv_stride_page, kv_stride_tok;
  int32_t kv_fp8;
  int32_t q_fp8;                 // E4M3 q codes (kv_fp8 too); q_scale folds into scale_log2
  float kv_scale;
  const int32_t *seq_lens;
  const int32_t *block_table;
  int32_t block_table_stride;
  int32_t batch, q_len, num_heads;
  int32_t page_shift;
  int32_t fold, q_groups, rows;  // rows per unit: num_heads * fold, or up to 128 packed rows
  int32_t packed;                // rows numbered t * num_heads + h across the q_len tokens
  int32_t num_splits, split_tokens;
  float scale_log2;
  int32_t causal;
  int32_t window_left;           // keys of context before the query block; -1: full history
  void *o;
  float *lse;
  float *o_parts;
  float *lse_parts;
};

struct MergeArgs {
  const float *o_parts;          // [S, R, Dv]
  const float *lse_parts;        // [S, R]
  int32_t num_splits;
  int64_t num_rows;
  int32_t head_dim_v;
  void *o;                       // [R, Dv]
  int32_t o_bf16;                // 1: bf16 output, 0: fp32
  float *lse;                    // optional [R]
  // key ranges of the GQA decode (key_ranges > 0): a row's pieces are found
  // from seq_lens as the split kernel cut them; rows of a request that lies
  // inside one range are final already and left alone
  int32_t key_ranges;
  const int32_t *seq_lens;
  int32_t batch, q_len, window_left;
  int32_t rows_per_request;      // q_len * Hq
};

struct PrefillArgs {
  const void *q;
  int64_t q_stride_tok, q_stride_head;
  const void *k, *v;
  int64_t k_stride_page, k_stride_tok, k_stride_head;
  int64_t v_stride_page, v_stride_tok, v_stride_head;
  const int32_t *cu_seqlens_q;
  const int32_t *cu_seqlens_kv;
  const int32_t *seq_lens_kv;
  const int32_t *block_table;    // null: dense
  int32_t block_table_stride;
  int32_t page_shift;
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t max_seqlen_q, max_seqlen_kv;
  int32_t q_tiles;               // ceil(max_seqlen_q / rows per workgroup)
  float scale_log2;
  int32_t causal;
  int32_t window_left;           // keys of context before the query block; -1: full history
  int32_t fp8;                   // 1: E4M3 q/k/v codes (scale_log2 carries q_scale * k_scale)
  float v_scale;                 // FP8: V dequantisation scale (1 for bf16)
  int32_t total_q;               // query tokens of all requests (rows of the partials / Hq)
  int32_t kv_splits;             // workgroups per query tile along the keys (1: no partials)
  int32_t split_tokens;          // keys per split, a multiple of 64
  float *o_parts;                // kv_splits > 1: [S, total_q * Hq, Dv] normalised partial outputs
  float *lse_parts;              // kv_splits > 1: [S, total_q * Hq] base-2 LSE of each split
  void *o;
  int64_t o_stride_tok, o_stride_head;
  float *lse;
};

// K/V cache append, validated: row of token i = layer_base + max(slot[i], 0).
struct CacheAppendArgs {
  const void *k_new, *v_new;     // bf16; v_new null: K only
  int64_t k_new_stride_tok, k_new_stride_head;
  int64_t v_new_stride_tok, v_new_stride_head;
  void *k_cache, *v_cache;
  int64_t k_stride_page, k_stride_tok, k_stride_head;
  int64_t v_stride_page, v_stride_tok, v_stride_head;
  int32_t fp8;                   // 1: E4M3 codes, 0: bf16
  float k_scale, v_scale;
  const int64_t *slot_mapping;
  int64_t layer_base_rows, num_cache_rows;
  int32_t num_tokens, num_kv_heads, head_dim_k, head_dim_v;
  int32_t page_shift;
};

// MLA K/V pack: K = concat(k_nope[t, h], k_rope[t]) and V, quantised to E4M3.
struct MlaPackArgs {
  const void *k_nope, *k_rope, *v;
  int64_t k_nope_stride_tok, k_nope_stride_head, k_rope_stride_tok;
  int64_t v_stride_tok, v_stride_head;
  void *k_out, *v_out;
  int64_t k_out_stride_tok, k_out_stride_head, v_out_stride_tok, v_out_stride_head;
  float k_scale, v_scale;
  int32_t num_tokens, num_heads, d_nope, d_rope, d_v;
};

// Launchers; each returns hipSuccess or the launch error.
// Waves of the GQA decode kernel one CU holds at once (its occupancy by
// registers), for the planner.
int decode_gqa_waves_per_cu(int head_dim, bool ext);
hipError_t launch_decode_gqa(const DecodeGqaArgs &a, hipStream_t stream);
hipError_t launch_decode_mla(const DecodeMlaArgs &a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_prefill_fp8(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_cache_append(const CacheAppendArgs &a, hipStream_t stream);
hipError_t launch_mla_kv_pack(const MlaPackArgs &a, hipStream_t stream);

// Kernel geometry the planner needs.
constexpr int kGqaRowsPerTile = 16;   // MFMA N rows of the GQA decode kernel
constexpr int kGqaTileTokens = 32;    // keys per wave iteration

constexpr int kMlaRows = 128;         // folded rows of the MLA decode kernel
constexpr int kMlaTileTokens = 32;
constexpr int kMaxSplits = 256;
constexpr int kDefaultCUs = 256;      // MI355X compute units: the plan when no device is visible
constexpr int kMaxDevices = 64;       // device ordinals whose CU count is cached
constexpr float kLog2eHost = 1.4426950408889634f;

}  // namespace attn
