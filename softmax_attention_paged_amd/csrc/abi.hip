// C-ABI entry points: host-side validation, planning and dispatch.
//
// Nothing here touches device memory: arguments are checked from host
// scalars and pointer values only, the plan depends only on host scalars
// (never on device seq_lens), and the kernels are enqueued on the caller's
// stream. That keeps every call free of synchronisation and capturable.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "attn_internal.h"

namespace {

thread_local char g_last_error[256] = "";

attn_status_t fail(attn_status_t s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

attn_status_t ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, asked of the runtime once per device
// and cached (an attribute query: no synchronisation, no device memory).
// Without a visible device (planning on a host with no GPU) the plan is made
// for the 256 CUs of an MI355X; a failed query's error is cleared so that it
// cannot surface as a later launch's error.
int num_cus() {
  static std::atomic<int> cached[attn::kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= attn::kMaxDevices) {
    (void)hipGetLastError();
    return attn::kDefaultCUs;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return attn::kDefaultCUs;
  }
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool is_mla_shape(const attn_decode_params *p) {
  return p->head_dim_qk == 576 && p->head_dim_v == 512;
}

// Largest F dividing q_len with rows_per_head * F <= capacity ("TokenSpeed-MLA",
// section "Key Optimization ... Group q_seqlen and num_heads into BMM1 M").
int fold_factor(int heads, int q_len, int capacity) {
  int best = 1;
  for (int f = 1; f <= q_len; ++f)
    if (q_len % f == 0 && heads * f <= capacity) best = f;
  return best;
}

// Keys a unit may have to walk: the whole history, or with a window the
// q_len block plus window_left keys of context, plus up to 31 keys of tile
// alignment before the window's start.
int window_span(const attn_decode_params *p) {
  if (!p->window_enabled) return p->max_seq_len;
  return (int)std::min<int64_t>(p->max_seq_len, (int64_t)p->window_left + p->q_len + 31);
}

struct DecodePlan {
  bool mla;
  int group, fold, q_groups, rows, splits, split_tokens;
  int key_ranges;          // > 0: the GQA decode cuts the batch's tiles into this many ranges
  int64_t units;
  size_t workspace;
};

// Shortest key range the planner cuts (tiles of 32 keys): a range pays a
// query load and an output write per request it touches. Graph replays on one
// GPU (batches 1-64, bounds 512-4096 keys, 40/8 heads at D 128 and 8/2 at
// D 64): a minimum of 2 tiles ran 0.61-1.0 of the time of a minimum of 8
// (4 requests <= 1024 keys at D 128: 13.1 against 20.6 us), 4 tiles in
// between; batches that fill the range cap (the 64 x 8192 decode) unchanged.
constexpr int kMinRangeTiles = 2;
// Waves per CU the key ranges are cut for: two per SIMD. Measured on the
// 64-request decode (lengths uniform on 256..8192, Hkv 8, D 128, three
// resident per SIMD): 7, 7.5, 8, 8.5, 9 and 12 waves per CU ran 0.1905,
// 0.1904, 0.1894, 0.1929, 0.1921 and 0.198 ms per call: fewer concurrent
// streams read the paged pool more efficiently, down to the point where
// too few requests are in flight.
constexpr int kRangeWavesPerCU = 8;
// Longest walk (tiles of 32 keys) for which a decode runs unsplit when every
// unit is resident at once: one launch, no partials. Graph replays on one
// GPU (batches 1-64, 8/2 heads at D 64 and 40/8 at D 128, lengths from half
// the longest up to it): up to 256 keys the unsplit launch took 3.9-24.5 us
// against 4.9-27.5 us for key ranges and their merge (0.28-0.90 of the
// time); from 512 keys the key ranges were faster (1.1-5.4x). Measured
// against key ranges of at least 8 tiles; the 2-tile minimum above is
// faster at these sizes, so the limit may be lower at D 128.
constexpr int kUnsplitMaxTiles = 8;

attn_status_t validate_decode(const attn_decode_params *p, bool check_pointers) {
  if (!p) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0) return fail(ATTN_ERR_INVALID_ARG, "batch %d < 0", p->batch);
  if (p->q_len < 1 || p->q_len > 4)
    return fail(ATTN_ERR_UNSUPPORTED, "q_len %d outside 1..4", p->q_len);
  if (p->total_kv_tokens < 0) return fail(ATTN_ERR_INVALID_ARG, "total_kv_tokens < 0");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_q_heads % p->num_kv_heads)
    return fail(ATTN_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                p->num_q_heads, p->num_kv_heads);
  if (!pow2(p->page_size) || p->page_size < 16)
    return fail(ATTN_ERR_UNSUPPORTED, "page_size %d is not a power of two >= 16", p->page_size);
  if (p->max_seq_len < 0) return fail(ATTN_ERR_INVALID_ARG, "max_seq_len %d < 0", p->max_seq_len);
  // No request has a key (max_seq_len == 0): every row is empty (O = 0, LSE
  // = -inf) and neither the caches nor the block table are read, so they may
  // be empty and NULL.
  const bool any_keys = p->max_seq_len > 0;
  if (any_keys && p->num_pages < 1) return fail(ATTN_ERR_INVALID_ARG, "num_pages %d < 1", p->num_pages);
  if ((int64_t)p->max_seq_len > (int64_t)p->num_pages * p->page_size)
    return fail(ATTN_ERR_INVALID_ARG, "max_seq_len %d exceeds num_pages * page_size", p->max_seq_len);
  if (p->block_table_stride < cdiv(p->max_seq_len, p->page_size))
    return fail(ATTN_ERR_INVALID_ARG, "block_table_stride %d < pages of max_seq_len (%lld)",
                p->block_table_stride, (long long)cdiv(p->max_seq_len, p->page_size));
  if (!std::isfinite(p->softmax_scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (p->causal != 0 && p->causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->num_splits < 0 || p->num_splits > attn::kMaxSplits)
    return fail(ATTN_ERR_INVALID_ARG, "num_splits %d outside 0..%d", p->num_splits, attn::kMaxSplits);
  if (p->window_enabled != 0 && p->window_enabled != 1)
    return fail(ATTN_ERR_INVALID_ARG, "window_enabled must be 0 or 1");
  if (p->window_enabled && p->window_left < 0)
    return fail(ATTN_ERR_INVALID_ARG, "window_left %d < 0", p->window_left);
  if (p->packed_q != 0 && p->packed_q != 1) return fail(ATTN_ERR_INVALID_ARG, "packed_q must be 0 or 1");

  const bool mla = is_mla_shape(p);
  if (mla) {
    if (p->num_kv_heads != 1)
      return fail(ATTN_ERR_UNSUPPORTED, "the 576/512 latent layout needs num_kv_heads == 1");
    if (p->kv_dtype != ATTN_BF16 && p->kv_dtype != ATTN_FP8_E4M3)
      return fail(ATTN_ERR_UNSUPPORTED, "latent KV must be bf16 or fp8 e4m3");
    if (p->k_cache != p->v_cache || p->k_stride_page != p->v_stride_page || p->k_stride_tok != p->v_stride_tok)
      return fail(ATTN_ERR_UNSUPPORTED, "the latent layout reads V from the K rows: pass the same cache and strides");
    if (p->num_q_heads > attn::kMlaRows)
      return fail(ATTN_ERR_UNSUPPORTED, "latent decode supports at most %d query heads", attn::kMlaRows);
    if (p->kv_dtype == ATTN_FP8_E4M3 &&
        (!(p->k_scale > 0.f) || !std::isfinite(p->k_scale) || p->k_scale != p->v_scale))
      return fail(ATTN_ERR_INVALID_ARG, "fp8 latent KV needs one finite positive scale (k_scale == v_scale)");
  } else {
    if (p->head_dim_qk != p->head_dim_v ||
        (p->head_dim_qk != 64 && p->head_dim_qk != 128 && p->head_dim_qk != 256))
      return fail(ATTN_ERR_UNSUPPORTED, "head dims (%d, %d) unsupported: need equal 64/128/256 or 576/512",
                  p->head_dim_qk, p->head_dim_v);
    if (p->kv_dtype != ATTN_BF16)
      return fail(ATTN_ERR_UNSUPPORTED, "GQA decode supports bf16 KV only");
    if (p->num_q_heads / p->num_kv_heads > attn::kGqaRowsPerTile)
      return fail(ATTN_ERR_UNSUPPORTED, "more than %d query heads per KV head", attn::kGqaRowsPerTile);
  }
  if (p->kv_dtype == ATTN_BF16 && (p->k_scale != 1.f || p->v_scale != 1.f))
    return fail(ATTN_ERR_INVALID_ARG, "k_scale and v_scale must be 1.0 for bf16 KV");
  if (p->q_dtype != ATTN_BF16 && p->q_dtype != ATTN_FP8_E4M3)
    return fail(ATTN_ERR_INVALID_ARG, "q_dtype must be ATTN_BF16 or ATTN_FP8_E4M3");
  if (p->q_dtype == ATTN_FP8_E4M3) {
    if (!mla || p->kv_dtype != ATTN_FP8_E4M3)
      return fail(ATTN_ERR_UNSUPPORTED, "fp8 q is supported with an MLA-shaped fp8 cache only");
    if (!(p->q_scale > 0.f) || !std::isfinite(p->q_scale))
      return fail(ATTN_ERR_INVALID_ARG, "fp8 q needs a finite positive q_scale");
  }

  if (p->batch == 0 || !check_pointers) return ok();
  if (!p->q || !p->seq_lens || !p->o || (any_keys && (!p->k_cache || !p->v_cache || !p->block_table)))
    return fail(ATTN_ERR_INVALID_ARG, "a required pointer (q, k_cache, v_cache, seq_lens, block_table, o) is NULL");
  if (!aligned16(p->q) || !aligned16(p->o)) return fail(ATTN_ERR_INVALID_ARG, "q, caches and o must be 16-byte aligned");
  if (!any_keys) return ok();
  if (!aligned16(p->k_cache) || !aligned16(p->v_cache))
    return fail(ATTN_ERR_INVALID_ARG, "q, caches and o must be 16-byte aligned");
  const int esz = (p->kv_dtype == ATTN_FP8_E4M3) ? 1 : 2;
  const int64_t strides[6] = {p->k_stride_page, p->k_stride_tok, p->k_stride_head,
                              p->v_stride_page, p->v_stride_tok, p->v_stride_head};
  for (int i = 0; i < 6; ++i) {
    if (strides[i] < 0 || (strides[i] * esz) % 16)
      return fail(ATTN_ERR_INVALID_ARG, "cache strides must be non-negative and multiples of 16 bytes");
  }
  if (p->k_stride_tok < 1 || p->k_stride_page < 1 || p->v_stride_tok < 1 || p->v_stride_page < 1)
    return fail(ATTN_ERR_INVALID_ARG, "cache page and token strides must be positive");
  return ok();
}

DecodePlan plan_decode(const attn_decode_params *p) {
  DecodePlan pl{};
  pl.mla = is_mla_shape(p);
  pl.group = p->num_q_heads / p->num_kv_heads;
  const int capacity = pl.mla ? attn::kMlaRows : attn::kGqaRowsPerTile;
  if (p->packed_q) {
    // continuous t * G + g rows in tiles of `capacity`, only the last one partial
    // ("TokenSpeed-MLA", packed-query paragraph)
    const int total = pl.group * p->q_len;
    pl.fold = 1;
    pl.rows = std::min(capacity, total);
    pl.q_groups = (int)cdiv(total, pl.rows);
  } else {
    pl.fold = fold_factor(pl.group, p->q_len, capacity);
    pl.q_groups = p->q_len / pl.fold;
    pl.rows = pl.group * pl.fold;
  }
  const int64_t base_units = (int64_t)p->batch * p->num_kv_heads * pl.q_groups;
  const int tile = pl.mla ? attn::kMlaTileTokens : attn::kGqaTileTokens;
  const int cus = num_cus();
  int splits = 0;
  if (p->num_splits > 0) {
    splits = p->num_splits;
  } else if (pl.mla) {
    // MFMA-bound, one workgroup per CU: the launch takes ceil(U S / CUs)
    // rounds of units 1/S as long, and each split adds its own prologue,
    // epilogue and merge work (about 0.5 % of a unit per split, from the
    // 80K-key timings: 16 splits = one round 0.426 ms, 32 = two rounds
    // 0.457 ms, 24 = a round and a half 0.551 ms). Take the S that
    // minimises ceil(U S / CUs) / S * (1 + S / 200), the smallest on ties;
    // no split shorter than 1024 keys.
    const int64_t u = base_units > 0 ? base_units : 1;
    const int64_t by_len = std::max<int64_t>(1, std::min<int64_t>(cdiv(window_span(p), 1024), attn::kMaxSplits));
    double best = 0.0;
    splits = 1;
    for (int64_t s = 1; s <= by_len; ++s) {
      const double cost = (double)cdiv(u * s, cus) / (double)s * (1.0 + (double)s / 200.0);
      if (s == 1 || cost < best * 0.999) {
        best = cost;
        splits = (int)s;
      }
    }
  } else {
    // HBM-bound. Key ranges: the batch's tiles cut evenly over the waves
    // the CUs hold, every wave resident from the start and streaming the
    // same bytes. The kernels scan seq_lens on the device (up to
    // kKeyRangeMaxBatch requests), so the plan needs no lengths; the host
    // total, when given, only caps the range count for small batches.
    const bool ext = p->window_enabled || p->packed_q;
    const int span = window_span(p);
    const int64_t req_tiles = cdiv(std::max(span, 1), tile) + 1;   // a request's tiles, window alignment included
    const int64_t resident = (int64_t)cus * attn::decode_gqa_waves_per_cu(p->head_dim_qk, ext);
    if (cdiv(std::max(span, 1), tile) <= kUnsplitMaxTiles && base_units <= resident) {
      // short requests: the key ranges' scans of seq_lens and the merge
      // launch cost more than the balance they buy
      splits = 1;
    } else if (p->batch <= attn::kKeyRangeMaxBatch && (int64_t)p->batch * req_tiles < (int64_t(1) << 30)) {
      const int64_t per = (int64_t)p->num_kv_heads * pl.q_groups;
      const int64_t slots = (int64_t)cus * std::min(kRangeWavesPerCU, attn::decode_gqa_waves_per_cu(p->head_dim_qk, ext));
      int64_t upper = (int64_t)p->batch * req_tiles;
      if (p->total_kv_tokens > 0) upper = std::min<int64_t>(upper, cdiv(p->total_kv_tokens, tile) + p->batch);
      const int64_t k = std::max<int64_t>(
          1, std::min<int64_t>({slots / per, (int64_t)attn::kMaxKeyRanges, cdiv(upper, kMinRangeTiles)}));
      pl.key_ranges = (int)k;
      pl.splits = 0;
      pl.split_tokens = 0;
      pl.units = k * per;
      const int64_t rows_req = (int64_t)p->q_len * p->num_q_heads;
      pl.workspace = k > 1 ? (size_t)(k + p->batch) * rows_req * (p->head_dim_v + 1) * sizeof(float) : 0;
      return pl;
    }
    // Otherwise one single-wave unit per (request, KV head, q-group, split).
    if (splits == 0 && p->total_kv_tokens > 0) {
      // With the host's total of the keys: the split length L for which every
      // unit is resident at once. A request walking n keys has at most
      // n / L + 1 units per (KV head, q-group), so with
      // (total / L + batch) * Hkv * q_groups <= the waves the CUs hold, the
      // launch is one round. Measured on three 64-request decodes (lengths
      // uniform on 256..8192, Hkv 8, D 128): 0.194-0.204 ms against
      // 0.203-0.213 ms for the fixed rule below; one more split than fits
      // (a few units in a second round) costs 20-30 %.
      const int64_t slots = (int64_t)cus * attn::decode_gqa_waves_per_cu(p->head_dim_qk, ext);
      const int64_t room = slots / ((int64_t)p->num_kv_heads * pl.q_groups) - p->batch;
      if (room > 0 && span > 0) {
        const int64_t total = std::min<int64_t>(p->total_kv_tokens, (int64_t)p->batch * span);
        int64_t st = std::max<int64_t>(256, cdiv(cdiv(total, room), tile) * tile);
        st = std::max<int64_t>(st, cdiv(cdiv(span, attn::kMaxSplits), tile) * tile);
        pl.splits = (int)std::max<int64_t>(1, cdiv(span, st));
        pl.split_tokens = (int)std::min<int64_t>(st, cdiv(span, tile) * tile);
        splits = -1;   // split length fixed above
      }
    }
    if (splits == 0) {
      // Otherwise many small units so ragged lengths balance across 256 CUs,
      // but no split shorter than 256 keys. 44 units per CU: from interleaved
      // median timings of three 64-request decodes (lengths uniform on
      // 256..8192, Hkv 8, D 128), 22 splits of 384 keys ran 5-6 % faster than
      // 16 of 512 (and than 18-20), while 23 of 352 ran 6-9 % slower.
      const int64_t want = cdiv(44 * cus, base_units > 0 ? base_units : 1);
      const int64_t by_len = cdiv(window_span(p), 256);
      splits = (int)std::max<int64_t>(1, std::min<int64_t>({want, by_len, attn::kMaxSplits}));
    }
  }
  // Split length: a whole number of tiles; then keep only non-empty splits of
  // the longest request. With a window, splits cover each request's window
  // (from its tile-aligned start), so the walk and the split count track the
  // window rather than the cache.
  const int span = window_span(p);
  if (splits > 0) {
    int64_t split_tokens = cdiv(std::max(span, 1), splits);
    split_tokens = cdiv(split_tokens, tile) * tile;
    pl.splits = (int)std::max<int64_t>(1, cdiv(span, split_tokens));
    pl.split_tokens = (int)split_tokens;
  }
  splits = pl.splits;
  pl.units = base_units * splits;
  const int64_t rows_total = (int64_t)p->batch * p->q_len * p->num_q_heads;
  pl.workspace = splits > 1 ? (size_t)splits * rows_total * (p->head_dim_v + 1) * sizeof(float) : 0;
  return pl;
}


// Query rows per prefill workgroup and workgroups a CU holds at once, by
// head dim: the D = 128 kernel runs eight waves (256 rows, one workgroup per
// CU), the others four (128 rows; two workgroups per CU at D = 64).
int prefill_rows_per_wg(int d) { return d == 128 ? 256 : 128; }
int prefill_wgs_per_cu(int d) { return d == 64 ? 2 : 1; }

// shapes_only: the checks a workspace query makes (no pointers or strides).
attn_status_t validate_prefill(const attn_prefill_params *p, bool shapes_only = false) {
  if (!p) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0) return fail(ATTN_ERR_INVALID_ARG, "batch %d < 0", p->batch);
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_q_heads % p->num_kv_heads)
    return fail(ATTN_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                p->num_q_heads, p->num_kv_heads);
  if (p->qkv_dtype != ATTN_BF16 && p->qkv_dtype != ATTN_FP8_E4M3)
    return fail(ATTN_ERR_UNSUPPORTED, "prefill qkv_dtype must be bf16 or fp8 e4m3");
  const bool fp8 = p->qkv_dtype == ATTN_FP8_E4M3;
  if (fp8) {
    if (p->head_dim_qk != 192 || p->head_dim_v != 128)
      return fail(ATTN_ERR_UNSUPPORTED, "FP8 prefill head dims (%d, %d) unsupported: need (192, 128)",
                  p->head_dim_qk, p->head_dim_v);
    if (p->block_table) return fail(ATTN_ERR_UNSUPPORTED, "FP8 prefill reads dense K/V only");
    for (float sc : {p->q_scale, p->k_scale, p->v_scale})
      if (!(std::isfinite(sc) && sc > 0.f)) return fail(ATTN_ERR_INVALID_ARG, "FP8 scales must be finite and > 0");
  } else if (p->head_dim_qk != p->head_dim_v ||
             (p->head_dim_qk != 64 && p->head_dim_qk != 128 && p->head_dim_qk != 256)) {
    return fail(ATTN_ERR_UNSUPPORTED, "prefill head dims (%d, %d) unsupported: need equal 64/128/256",
                p->head_dim_qk, p->head_dim_v);
  }
  if (p->max_seqlen_q < 0 || p->max_seqlen_kv < 0)
    return fail(ATTN_ERR_INVALID_ARG, "max_seqlen_q/max_seqlen_kv must be >= 0");
  if (p->kv_splits < 0 || p->kv_splits > attn::kMaxSplits)
    return fail(ATTN_ERR_INVALID_ARG, "kv_splits %d outside 0..%d", p->kv_splits, attn::kMaxSplits);
  if (p->total_q < 0) return fail(ATTN_ERR_INVALID_ARG, "total_q < 0");
  if (!std::isfinite(p->softmax_scale)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (p->causal != 0 && p->causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->window_enabled != 0 && p->window_enabled != 1)
    return fail(ATTN_ERR_INVALID_ARG, "window_enabled must be 0 or 1");
  if (p->window_enabled && p->window_left < 0)
    return fail(ATTN_ERR_INVALID_ARG, "window_left %d < 0", p->window_left);
  const bool paged = p->block_table != nullptr;
  // No request has a key (max_seqlen_kv == 0): every row is empty (O = 0,
  // LSE = -inf) and K/V are never read, so they may be empty and NULL.
  const bool any_keys = p->max_seqlen_kv > 0;
  if (paged) {
    if (!pow2(p->page_size) || p->page_size < 16)
      return fail(ATTN_ERR_UNSUPPORTED, "page_size %d is not a power of two >= 16", p->page_size);
    if (any_keys && p->num_pages < 1) return fail(ATTN_ERR_INVALID_ARG, "num_pages %d < 1", p->num_pages);
    if ((int64_t)p->max_seqlen_kv > (int64_t)p->num_pages * p->page_size)
      return fail(ATTN_ERR_INVALID_ARG, "max_seqlen_kv exceeds num_pages * page_size");
    if (p->block_table_stride < cdiv(p->max_seqlen_kv, p->page_size))
      return fail(ATTN_ERR_INVALID_ARG, "block_table_stride %d < pages of max_seqlen_kv", p->block_table_stride);
  }
  if (shapes_only || p->batch == 0 || p->max_seqlen_q == 0) return ok();
  if (!p->q || !p->cu_seqlens_q || !p->o || (any_keys && (!p->k || !p->v)))
    return fail(ATTN_ERR_INVALID_ARG, "a required pointer (q, k, v, cu_seqlens_q, o) is NULL");
  if (paged ? !p->seq_lens_kv : !p->cu_seqlens_kv)
    return fail(ATTN_ERR_INVALID_ARG, paged ? "paged mode needs seq_lens_kv" : "dense mode needs cu_seqlens_kv");
  if (!aligned16(p->q) || !aligned16(p->o) || (any_keys && (!aligned16(p->k) || !aligned16(p->v))))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  // every stride a multiple of 16 bytes (elements of 2 bytes, or of 1 byte for FP8 inputs)
  const int64_t in_bytes = fp8 ? 1 : 2;
  const int64_t kv_strides[] = {p->k_stride_tok * in_bytes, p->k_stride_head * in_bytes, p->v_stride_tok * in_bytes,
                                p->v_stride_head * in_bytes, paged ? p->k_stride_page * in_bytes : 16,
                                paged ? p->v_stride_page * in_bytes : 16};
  const int64_t strides[] = {p->q_stride_tok * in_bytes, p->q_stride_head * in_bytes, p->o_stride_tok * 2,
                             p->o_stride_head * 2};
  for (int64_t st : strides)
    if (st < 0 || st % 16) return fail(ATTN_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  if (any_keys)
    for (int64_t st : kv_strides)
      if (st < 0 || st % 16) return fail(ATTN_ERR_INVALID_ARG, "strides must be non-negative multiples of 16 bytes");
  if (p->q_stride_tok < 1 || p->o_stride_tok < 1 || (any_keys && (p->k_stride_tok < 1 || p->v_stride_tok < 1)))
    return fail(ATTN_ERR_INVALID_ARG, "token strides must be positive");
  return ok();
}

// Key splits of a bf16 prefill: workgroups per query tile along the keys.
// Workgroups are counted from total_q (query tiles of prefill_rows_per_wg /
// gh tokens, times the head groups) against the CUs' slots. Measured on
// 80K-key paged prefills (with the four-wave D = 128 kernel, 128-row
// workgroups, two per CU: the same ratios of workgroups to slots as the
// eight-wave kernel's 256-row workgroups, one per CU):
//   - at most half a round (under one workgroup per slot pair): split by the
//     largest power of two that keeps the launch within one round (one
//     512-query chunk, 128 workgroups: 1.56 -> 0.67 ms at four splits);
//   - more than one round with a last round at most three quarters full:
//     four splits (768 workgroups over 512 slots: 4.67 -> 4.40 ms);
//   - otherwise unsplit: between half and one round, or whole rounds, the
//     splits cost more than they balance (384 workgroups: 1.68 ms unsplit,
//     1.75-1.81 split).
// No split is shorter than 8192 keys. Splits are numbered slowest, so the
// workgroups running together still share each K/V tile they stream as
// widely in L2 as without splits.
struct PrefillPlan {
  int splits;
  int split_tokens;
  size_t workspace;
};

bool prefill_o_contiguous(const attn_prefill_params *p) {
  return p->o_stride_head == p->head_dim_v && p->o_stride_tok == (int64_t)p->num_q_heads * p->head_dim_v;
}

PrefillPlan plan_prefill(const attn_prefill_params *p) {
  PrefillPlan pl{1, 0, 0};
  if (p->qkv_dtype != ATTN_BF16 || p->total_q <= 0 || !prefill_o_contiguous(p) || p->max_seqlen_kv <= 0 || p->batch <= 0 ||
      p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads)
    return pl;
  int splits = p->kv_splits;
  if (splits <= 0) {
    const int group = p->num_q_heads / p->num_kv_heads;
    const int gh = (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
    const int64_t units = std::max<int64_t>(1, cdiv(p->total_q, prefill_rows_per_wg(p->head_dim_qk) / gh)) *
                          (p->num_q_heads / gh);
    const int64_t slots = (int64_t)num_cus() * prefill_wgs_per_cu(p->head_dim_qk);
    int64_t sp = 1;
    if (2 * units <= slots) {
      while (2 * sp * units <= slots) sp *= 2;
    } else if (units > slots && units < 4 * slots && units % slots != 0 && 4 * (units % slots) <= 3 * slots) {
      sp = 4;
    }
    splits = (int)std::max<int64_t>(1, std::min<int64_t>(sp, p->max_seqlen_kv / 8192));
  }
  splits = std::min(splits, attn::kMaxSplits);
  if (splits <= 1) return pl;
  int64_t st = cdiv(cdiv(p->max_seqlen_kv, splits), 64) * 64;
  splits = (int)cdiv(p->max_seqlen_kv, st);
  if (splits <= 1) return pl;
  pl.splits = splits;
  pl.split_tokens = (int)st;
  pl.workspace = (size_t)splits * p->total_q * p->num_q_heads * (p->head_dim_v + 1) * sizeof(float);
  return pl;
}

}  // namespace

extern "C" {

const char *attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE_TOO_SMALL: return "ATTN_ERR_WORKSPACE_TOO_SMALL";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "ATTN_ERR_UNKNOWN";
}

const char *attn_last_error(void) { return g_last_error; }

attn_status_t attn_decode_plan(const attn_decode_params *p, attn_decode_plan_info *info) {
  if (!info) return fail(ATTN_ERR_INVALID_ARG, "info is NULL");
  attn_status_t st = validate_decode(p, false);
  if (st != ATTN_OK) return st;
  const DecodePlan pl = plan_decode(p);
  info->group = pl.group;
  info->fold = pl.fold;
  info->q_groups = pl.q_groups;
  info->rows_per_unit = pl.rows;
  info->num_splits = pl.splits;
  info->split_tokens = pl.split_tokens;
  info->num_units = pl.units;
  info->workspace_bytes = pl.workspace;
  info->key_ranges = pl.key_ranges;
  return ok();
}

size_t attn_decode_workspace_size(const attn_decode_params *p) {
  if (validate_decode(p, false) != ATTN_OK) return 0;
  return plan_decode(p).workspace;
}

}  // extern "C"

namespace {

// Which kernels of a decode call to enqueue.
enum DecodePhase { kPhaseSplit = 1, kPhaseMerge = 2, kPhaseBoth = 3 };

// The split kernel and, when the plan has partials, the merge, for a
// validated call whose partials go to `workspace`.
attn_status_t decode_enqueue(const attn_decode_params *p, const DecodePlan &pl, void *workspace,
                             hipStream_t stream, int phase = kPhaseBoth) {
  const int64_t rows_total = (int64_t)p->batch * p->q_len * p->num_q_heads;
  // partial slots: S per row, or key_ranges + batch per row of a request
  const int64_t part_rows = pl.key_ranges > 0 ? (int64_t)(pl.key_ranges + p->batch) * p->q_len * p->num_q_heads
                                              : (int64_t)pl.splits * rows_total;
  float *o_parts = static_cast<float *>(workspace);
  float *lse_parts = pl.workspace > 0 ? o_parts + (size_t)part_rows * p->head_dim_v : nullptr;
  const float scale_log2 = p->softmax_scale * attn::kLog2eHost;
  hipError_t err = hipSuccess;
  if (!(phase & kPhaseSplit)) {
    // merge only
  } else if (pl.mla) {
    attn::DecodeMlaArgs a{};
    a.q = p->q;
    a.kv_cache = p->k_cache;
    a.kv_stride_page = p->k_stride_page;
    a.kv_stride_tok = p->k_stride_tok;
    a.kv_fp8 = p->kv_dtype == ATTN_FP8_E4M3;
    a.q_fp8 = p->q_dtype == ATTN_FP8_E4M3;
    // FP8 codes are used as stored: k_scale folds into the score scale,
    // v_scale into the output normalisation.
    a.kv_scale = a.kv_fp8 ? p->v_scale : 1.0f;
    a.seq_lens = p->seq_lens;
    a.block_table = p->block_table;
    a.block_table_stride = p->block_table_stride;
    a.batch = p->batch;
    a.q_len = p->q_len;
    a.num_heads = p->num_q_heads;
    a.page_shift = log2i(p->page_size);
    a.fold = pl.fold;
    a.q_groups = pl.q_groups;
    a.rows = pl.rows;
    a.packed = p->packed_q;
    a.num_splits = pl.splits;
    a.split_tokens = pl.split_tokens;
    a.scale_log2 = (a.kv_fp8 ? scale_log2 * p->k_scale : scale_log2) * (a.q_fp8 ? p->q_scale : 1.f);
    a.causal = p->causal;
    a.window_left = p->window_enabled ? p->window_left : -1;
    a.o = p->o;
    a.lse = p->lse;
    a.o_parts = o_parts;
    a.lse_parts = lse_parts;
    err = attn::launch_decode_mla(a, stream);
  } else {
    attn::DecodeGqaArgs a{};
    a.q = p->q;
    a.k_cache = p->k_cache;
    a.v_cache = p->v_cache;
    a.k_stride_page = p->k_stride_page;
    a.k_stride_tok = p->k_stride_tok;
    a.k_stride_head = p->k_stride_head;
    a.v_stride_page = p->v_stride_page;
    a.v_stride_tok = p->v_stride_tok;
    a.v_stride_head = p->v_stride_head;
    a.seq_lens = p->seq_lens;
    a.block_table = p->block_table;
    a.block_table_stride = p->block_table_stride;
    a.batch = p->batch;
    a.q_len = p->q_len;
    a.num_q_heads = p->num_q_heads;
    a.num_kv_heads = p->num_kv_heads;
    a.head_dim = p->head_dim_qk;
    a.page_shift = log2i(p->page_size);
    a.group = pl.group;
    a.fold = pl.fold;
    a.q_groups = pl.q_groups;
    a.rows = pl.rows;
    a.packed = p->packed_q;
    a.num_splits = pl.splits;
    a.split_tokens = pl.split_tokens;
    a.key_ranges = pl.key_ranges;
    a.scale_log2 = scale_log2;
    a.causal = p->causal;
    a.window_left = p->window_enabled ? p->window_left : -1;
    a.o = p->o;
    a.lse = p->lse;
    a.o_parts = o_parts;
    a.lse_parts = lse_parts;
    err = attn::launch_decode_gqa(a, stream);
  }
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "split kernel launch: %s", hipGetErrorString(err));
  if ((phase & kPhaseMerge) && pl.workspace > 0) {
    attn::MergeArgs m{};
    m.o_parts = o_parts;
    m.lse_parts = lse_parts;
    m.num_splits = pl.splits;
    m.num_rows = rows_total;
    m.head_dim_v = p->head_dim_v;
    m.o = p->o;
    m.o_bf16 = 1;
    m.lse = p->lse;
    m.key_ranges = pl.key_ranges;
    m.seq_lens = p->seq_lens;
    m.batch = p->batch;
    m.q_len = p->q_len;
    m.window_left = p->window_enabled ? p->window_left : -1;
    m.rows_per_request = p->q_len * p->num_q_heads;
    err = attn::launch_merge(m, stream);
    if (err != hipSuccess) return fail(ATTN_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(err));
  }
  return ok();
}

// Scratch of attn_decode_paged_noalloc, for callers that cannot allocate:
// one array per device, held by the loaded library until the process ends.
// In host code `scratch` names a host-side stand-in, never the device
// array: its device address is asked for once per device and kept in
// g_scratch (see scratch_ptr). Calls on one device share it, so calls that
// overlap on one device (different streams) race; nothing in it needs to
// start at zero (each split writes every partial the merge reads).
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::atomic<void *> g_scratch[attn::kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on
// that device with the device current (no allocation), or null with the
// error recorded.
void *scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= attn::kMaxDevices) {
    (void)hipGetLastError();
    fail(ATTN_ERR_HIP, "no current HIP device (or its ordinal is %d or more)", attn::kMaxDevices);
    return nullptr;
  }
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (err != hipSuccess || !ptr) {
    (void)hipGetLastError();
    fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(err));
    return nullptr;
  }
  g_scratch[dev].store(ptr, std::memory_order_release);
  return ptr;
}

attn_status_t decode_call(const attn_decode_params *p, hipStream_t stream, int phase) {
  attn_status_t st = validate_decode(p, true);
  if (st != ATTN_OK) return st;
  if (p->batch == 0) return ok();
  const DecodePlan pl = plan_decode(p);
  if (pl.workspace > 0) {
    if (!p->workspace || p->workspace_bytes < pl.workspace)
      return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", pl.workspace,
                  p->workspace ? p->workspace_bytes : (size_t)0);
    if (!aligned16(p->workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  return decode_enqueue(p, pl, p->workspace, stream, phase);
}

}  // namespace

extern "C" {

attn_status_t attn_decode_paged(const attn_decode_params *p, hipStream_t stream) {
  return decode_call(p, stream, kPhaseBoth);
}

attn_status_t attn_decode_paged_split(const attn_decode_params *p, hipStream_t stream) {
  return decode_call(p, stream, kPhaseSplit);
}

attn_status_t attn_decode_paged_merge(const attn_decode_params *p, hipStream_t stream) {
  return decode_call(p, stream, kPhaseMerge);
}

attn_status_t attn_decode_paged_noalloc(const attn_decode_params *p, hipStream_t stream) {
  attn_status_t st = validate_decode(p, true);
  if (st != ATTN_OK) return st;
  if (p->batch == 0) return ok();
  const DecodePlan pl = plan_decode(p);
  if (pl.workspace > kStaticScratchBytes)
    return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "the plan needs %zu bytes of partials; the static scratch holds %zu",
                pl.workspace, kStaticScratchBytes);
  void *ws = nullptr;
  if (pl.workspace > 0 && !(ws = scratch_ptr())) return ATTN_ERR_HIP;
  return decode_enqueue(p, pl, ws, stream);
}

attn_status_t attn_prefill(const attn_prefill_params *p, hipStream_t stream) {
  attn_status_t st = validate_prefill(p);
  if (st != ATTN_OK) return st;
  if (p->batch == 0 || p->max_seqlen_q == 0) return ok();
  attn::PrefillArgs a{};
  a.q = p->q;
  a.q_stride_tok = p->q_stride_tok;
  a.q_stride_head = p->q_stride_head;
  a.k = p->k;
  a.v = p->v;
  a.k_stride_page = p->k_stride_page;
  a.k_stride_tok = p->k_stride_tok;
  a.k_stride_head = p->k_stride_head;
  a.v_stride_page = p->v_stride_page;
  a.v_stride_tok = p->v_stride_tok;
  a.v_stride_head = p->v_stride_head;
  a.cu_seqlens_q = p->cu_seqlens_q;
  a.cu_seqlens_kv = p->cu_seqlens_kv;
  a.seq_lens_kv = p->seq_lens_kv;
  a.block_table = p->block_table;
  a.block_table_stride = p->block_table_stride;
  a.page_shift = p->block_table ? log2i(p->page_size) : 0;
  a.batch = p->batch;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.head_dim = p->head_dim_qk;
  a.max_seqlen_q = p->max_seqlen_q;
  a.max_seqlen_kv = p->max_seqlen_kv;
  a.q_tiles = (int)cdiv(p->max_seqlen_q, prefill_rows_per_wg(p->head_dim_qk));
  a.fp8 = p->qkv_dtype == ATTN_FP8_E4M3;
  // FP8: the dequantisation scales of q and k fold into the score scale and
  // v's into the final normalisation
  a.scale_log2 = p->softmax_scale * attn::kLog2eHost * (a.fp8 ? p->q_scale * p->k_scale : 1.f);
  a.v_scale = a.fp8 ? p->v_scale : 1.f;
  a.causal = p->causal;
  a.window_left = p->window_enabled ? p->window_left : -1;
  a.o = p->o;
  a.o_stride_tok = p->o_stride_tok;
  a.o_stride_head = p->o_stride_head;
  a.lse = p->lse;
  a.kv_splits = 1;
  if (p->kv_splits > 1) {
    // forced key splits: anything that keeps them from running is an error
    if (a.fp8) return fail(ATTN_ERR_UNSUPPORTED, "key splits are built for bf16 prefill only");
    if (p->total_q <= 0) return fail(ATTN_ERR_INVALID_ARG, "key splits need total_q (the rows of q)");
    if (!prefill_o_contiguous(p))
      return fail(ATTN_ERR_UNSUPPORTED, "key splits need a contiguous o [total_q, Hq, Dv]");
  }
  const PrefillPlan pl = plan_prefill(p);
  if (pl.splits > 1 && p->kv_splits > 1) {
    if (!p->workspace || p->workspace_bytes < pl.workspace)
      return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "%d key splits need %zu workspace bytes, got %zu", pl.splits,
                  pl.workspace, p->workspace ? p->workspace_bytes : (size_t)0);
    if (!aligned16(p->workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  if (pl.splits > 1 && p->workspace && p->workspace_bytes >= pl.workspace && aligned16(p->workspace)) {
    a.kv_splits = pl.splits;
    a.split_tokens = pl.split_tokens;
    a.total_q = p->total_q;
    a.o_parts = static_cast<float *>(p->workspace);
    a.lse_parts = a.o_parts + (size_t)pl.splits * p->total_q * p->num_q_heads * p->head_dim_v;
  }
  hipError_t err = a.fp8 ? attn::launch_prefill_fp8(a, stream) : attn::launch_prefill(a, stream);
  if (err == hipErrorNotSupported) return fail(ATTN_ERR_UNSUPPORTED, "no prefill kernel for this shape");
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(err));
  return ok();
}

size_t attn_prefill_workspace_size(const attn_prefill_params *p) {
  if (!p || validate_prefill(p, true) != ATTN_OK) return 0;
  return plan_prefill(p).workspace;
}

attn_status_t attn_merge_lse(const float *o_parts, const float *lse_parts, int32_t num_splits,
                             int64_t num_rows, int32_t head_dim_v, void *o, attn_dtype_t o_dtype,
                             float *lse_out, hipStream_t stream) {
  if (num_splits < 1 || num_splits > attn::kMaxSplits)
    return fail(ATTN_ERR_INVALID_ARG, "num_splits %d outside 1..%d", num_splits, attn::kMaxSplits);
  if (num_rows < 0) return fail(ATTN_ERR_INVALID_ARG, "num_rows < 0");
  if (head_dim_v < 4 || head_dim_v > 1024 || head_dim_v % 4)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim_v %d must be a multiple of 4 in 4..1024", head_dim_v);
  if (o_dtype != ATTN_BF16 && o_dtype != ATTN_FP32)
    return fail(ATTN_ERR_UNSUPPORTED, "merge output must be bf16 or fp32");
  if (num_rows == 0) return ok();
  if (!o_parts || !lse_parts || !o) return fail(ATTN_ERR_INVALID_ARG, "o_parts, lse_parts and o are required");
  if (!aligned16(o_parts) || !aligned16(o) || (o_dtype == ATTN_BF16 && head_dim_v % 8 && (reinterpret_cast<uintptr_t>(o) & 7)))
    return fail(ATTN_ERR_INVALID_ARG, "o_parts and o must be 16-byte aligned");
  attn::MergeArgs m{};
  m.o_parts = o_parts;
  m.lse_parts = lse_parts;
  m.num_splits = num_splits;
  m.num_rows = num_rows;
  m.head_dim_v = head_dim_v;
  m.o = o;
  m.o_bf16 = o_dtype == ATTN_BF16;
  m.lse = lse_out;
  hipError_t err = attn::launch_merge(m, stream);
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(err));
  return ok();
}

attn_status_t attn_cache_append(const attn_cache_append_params *p, hipStream_t stream) {
  if (!p) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->num_tokens < 0) return fail(ATTN_ERR_INVALID_ARG, "num_tokens < 0");
  if (p->num_kv_heads < 1) return fail(ATTN_ERR_INVALID_ARG, "num_kv_heads < 1");
  const bool has_v = p->v_new != nullptr;
  for (int d : {p->head_dim_k, has_v ? p->head_dim_v : 8})
    if (d < 8 || d > 1024 || d % 8) return fail(ATTN_ERR_UNSUPPORTED, "head dims must be multiples of 8 in 8..1024");
  if (p->cache_dtype != ATTN_BF16 && p->cache_dtype != ATTN_FP8_E4M3)
    return fail(ATTN_ERR_UNSUPPORTED, "cache_dtype must be bf16 or fp8 e4m3");
  const bool fp8 = p->cache_dtype == ATTN_FP8_E4M3;
  if (fp8) {
    if (!(std::isfinite(p->k_scale) && p->k_scale > 0.f) || (has_v && !(std::isfinite(p->v_scale) && p->v_scale > 0.f)))
      return fail(ATTN_ERR_INVALID_ARG, "fp8 scales must be finite and > 0");
  } else if (p->k_scale != 1.f || (has_v && p->v_scale != 1.f)) {
    return fail(ATTN_ERR_INVALID_ARG, "bf16 caches take scales of 1.0");
  }
  if (!pow2(p->page_size)) return fail(ATTN_ERR_INVALID_ARG, "page_size must be a power of two");
  if (p->layer_base_rows < 0 || p->num_cache_rows < 0)
    return fail(ATTN_ERR_INVALID_ARG, "layer_base_rows and num_cache_rows must be >= 0");
  if (p->num_tokens == 0) return ok();
  if (!p->k_new || !p->k_cache || !p->slot_mapping || (has_v && !p->v_cache))
    return fail(ATTN_ERR_INVALID_ARG, "k_new, k_cache, slot_mapping (and v_cache with v_new) are required");
  if ((reinterpret_cast<uintptr_t>(p->slot_mapping) & 7u) != 0)
    return fail(ATTN_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");
  // every 8-element chunk starts 16-byte aligned in the inputs, and 16-byte
  // (bf16) or 8-byte (fp8) aligned in the cache
  const uintptr_t cache_align = fp8 ? 7u : 15u;
  auto chunk_ok = [&](const void *ptr, uintptr_t mask, std::initializer_list<int64_t> strides) {
    if (reinterpret_cast<uintptr_t>(ptr) & mask) return false;
    for (int64_t st : strides)
      if (st < 0 || st % 8) return false;
    return true;
  };
  if (!chunk_ok(p->k_new, 15u, {p->k_new_stride_tok, p->k_new_stride_head}) ||
      (has_v && !chunk_ok(p->v_new, 15u, {p->v_new_stride_tok, p->v_new_stride_head})))
    return fail(ATTN_ERR_INVALID_ARG, "k_new/v_new need 16-byte aligned rows and non-negative strides that are multiples of 8");
  if (!chunk_ok(p->k_cache, cache_align, {p->k_stride_page, p->k_stride_tok, p->k_stride_head}) ||
      (has_v && !chunk_ok(p->v_cache, cache_align, {p->v_stride_page, p->v_stride_tok, p->v_stride_head})))
    return fail(ATTN_ERR_INVALID_ARG, "cache rows must be aligned to 8 elements with non-negative strides that are multiples of 8");
  attn::CacheAppendArgs a{};
  a.k_new = p->k_new;
  a.v_new = p->v_new;
  a.k_new_stride_tok = p->k_new_stride_tok;
  a.k_new_stride_head = p->k_new_stride_head;
  a.v_new_stride_tok = p->v_new_stride_tok;
  a.v_new_stride_head = p->v_new_stride_head;
  a.k_cache = p->k_cache;
  a.v_cache = p->v_cache;
  a.k_stride_page = p->k_stride_page;
  a.k_stride_tok = p->k_stride_tok;
  a.k_stride_head = p->k_stride_head;
  a.v_stride_page = p->v_stride_page;
  a.v_stride_tok = p->v_stride_tok;
  a.v_stride_head = p->v_stride_head;
  a.fp8 = fp8;
  a.k_scale = p->k_scale;
  a.v_scale = p->v_scale;
  a.slot_mapping = p->slot_mapping;
  a.layer_base_rows = p->layer_base_rows;
  a.num_cache_rows = p->num_cache_rows;
  a.num_tokens = p->num_tokens;
  a.num_kv_heads = p->num_kv_heads;
  a.head_dim_k = p->head_dim_k;
  a.head_dim_v = has_v ? p->head_dim_v : 0;
  a.page_shift = log2i(p->page_size);
  hipError_t err = attn::launch_cache_append(a, stream);
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "cache append launch: %s", hipGetErrorString(err));
  return ok();
}

attn_status_t attn_mla_kv_pack_fp8(const attn_mla_kv_pack_params *p, hipStream_t stream) {
  if (!p) return fail(ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->num_tokens < 0 || p->num_heads < 1) return fail(ATTN_ERR_INVALID_ARG, "num_tokens < 0 or num_heads < 1");
  if (p->d_nope < 8 || p->d_rope < 0 || p->d_v < 8 || p->d_nope % 8 || p->d_rope % 8 || p->d_v % 8 ||
      p->d_nope + p->d_rope > 4096 || p->d_v > 4096)
    return fail(ATTN_ERR_INVALID_ARG, "d_nope, d_v >= 8 and d_rope >= 0 must be multiples of 8 (<= 4096)");
  if (!(std::isfinite(p->k_scale) && p->k_scale > 0.f && std::isfinite(p->v_scale) && p->v_scale > 0.f))
    return fail(ATTN_ERR_INVALID_ARG, "scales must be finite and > 0");
  if (p->num_tokens == 0) return ok();
  if (!p->k_nope || !p->v || !p->k_out || !p->v_out || (p->d_rope > 0 && !p->k_rope))
    return fail(ATTN_ERR_INVALID_ARG, "k_nope, k_rope, v, k_out and v_out are required");
  auto ok_in = [](const void *ptr, std::initializer_list<int64_t> strides) {
    if (reinterpret_cast<uintptr_t>(ptr) & 15u) return false;
    for (int64_t st : strides)
      if (st < 0 || st % 8) return false;
    return true;
  };
  auto ok_out = [](const void *ptr, std::initializer_list<int64_t> strides) {
    if (reinterpret_cast<uintptr_t>(ptr) & 7u) return false;
    for (int64_t st : strides)
      if (st < 0 || st % 8) return false;
    return true;
  };
  if (!ok_in(p->k_nope, {p->k_nope_stride_tok, p->k_nope_stride_head}) || !ok_in(p->v, {p->v_stride_tok, p->v_stride_head}) ||
      (p->d_rope > 0 && !ok_in(p->k_rope, {p->k_rope_stride_tok})))
    return fail(ATTN_ERR_INVALID_ARG, "inputs need 16-byte aligned rows and non-negative strides that are multiples of 8");
  if (!ok_out(p->k_out, {p->k_out_stride_tok, p->k_out_stride_head}) || !ok_out(p->v_out, {p->v_out_stride_tok, p->v_out_stride_head}))
    return fail(ATTN_ERR_INVALID_ARG, "outputs need 8-byte aligned rows and non-negative strides that are multiples of 8");
  // the kernel addresses rows within a token with 24-bit multiplies
  for (int64_t st : {p->k_nope_stride_head, p->v_stride_head, p->k_out_stride_head, p->v_out_stride_head})
    if (st >= (int64_t(1) << 24) || int64_t(p->num_heads) * st + 4096 >= (int64_t(1) << 31))
      return fail(ATTN_ERR_UNSUPPORTED, "per-head strides must be below 2^24 elements and one token's rows below 2^31");
  if (p->num_heads >= (1 << 24)) return fail(ATTN_ERR_UNSUPPORTED, "num_heads must be below 2^24");
  attn::MlaPackArgs a{};
  a.k_nope = p->k_nope;
  a.k_rope = p->k_rope;
  a.v = p->v;
  a.k_nope_stride_tok = p->k_nope_stride_tok;
  a.k_nope_stride_head = p->k_nope_stride_head;
  a.k_rope_stride_tok = p->k_rope_stride_tok;
  a.v_stride_tok = p->v_stride_tok;
  a.v_stride_head = p->v_stride_head;
  a.k_out = p->k_out;
  a.v_out = p->v_out;
  a.k_out_stride_tok = p->k_out_stride_tok;
  a.k_out_stride_head = p->k_out_stride_head;
  a.v_out_stride_tok = p->v_out_stride_tok;
  a.v_out_stride_head = p->v_out_stride_head;
  a.k_scale = p->k_scale;
  a.v_scale = p->v_scale;
  a.num_tokens = p->num_tokens;
  a.num_heads = p->num_heads;
  a.d_nope = p->d_nope;
  a.d_rope = p->d_rope;
  a.d_v = p->d_v;
  hipError_t err = attn::launch_mla_kv_pack(a, stream);
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "MLA K/V pack launch: %s", hipGetErrorString(err));
  return ok();
}

}  // extern "C"
