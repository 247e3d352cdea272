// Paged GQA decode, split over the KV sequence, for gfx950.
//
// Work unit: one request b, one KV head with the G query heads that share it
// ("Writing Page Attention with PyPTO", section 1.3: one task is one batch row
// + one KV head + its query heads, so the KV pages are read once for all of
// them), the F query tokens folded with those heads into the MFMA row
// dimension ("TokenSpeed-MLA", section "Key Optimization ... Group q_seqlen
// and num_heads into BMM1 M"), and one KV split.
//
// A wave walks 32-key tiles of its unit and keeps a running max m, sums l
// and output o per row (the online recurrence of "Flywheel Attention",
// section 1, and "Writing Page Attention with PyPTO", section 6.3). Per tile:
//   - K and V rows are gathered through the block table into registers with
//     full-row loads (16 lanes per 256-byte row slice), both issued at the
//     top of the tile's iteration; the page of a 16-key half-tile is one
//     table entry (pages hold a power of two >= 16 keys), read once. K goes through the wave's LDS tile to the
//     MFMA A-operand layout (token = l % 16, 8 channels per lane), then V
//     takes the same tile.
//   - S^T = K Q^T on v_mfma_f32_16x16x32_bf16, so each lane ends up holding
//     8 scores of ONE row (l % 16): the softmax state is lane-local.
//   - Invalid keys (past the split, past the request, or above the causal
//     diagonal) get -inf before the max and exp ("Writing Page Attention
//     with PyPTO", section 6.2), and their V rows are zeroed, so NaN in page
//     tails cannot reach an FMA.
//   - P (rounded to bf16, RNE) feeds O^T += V^T P^T directly from the score
//     registers; V^T comes from a wave-private LDS copy of the V tile read
//     with ds_read_b64_tr_b16. Two row sums are kept: the rounded P that
//     multiplied V normalises O (so a constant V comes back exactly), and
//     the unrounded FP32 P gives the log-sum-exp.
// A unit that covers its request's whole key range writes bf16 O and the
// base-2 LSE; otherwise FP32 partials (O normalised over the unit's keys,
// LSE of those keys) that the merge kernel reduces ("TokenSpeed-MLA",
// section "Decode performance").
//
// Which keys a wave walks, one of two plans:
//   - key ranges (the planner's choice up to 512 requests): the 32-key
//     tiles of all requests, in request order, are cut into K ranges of
//     equal length, and range g is walked by Hkv * q_groups waves (one per
//     KV head and query group); a range that crosses request boundaries
//     walks one piece per request. Every wave streams the same bytes, so
//     the launch does not wait for the longest requests' last splits; K
//     gives two waves per SIMD. The kernel finds its pieces by scanning
//     seq_lens itself, so the host plan needs no lengths.
//   - per-request splits (forced split counts, larger batches): one unit
//     per (request, split).
// A workgroup is one wave. Workgroups are numbered with the query group,
// then the KV head, fastest: the units that read the per-head slices of the
// same token rows ([page, slot, head, dim] stores a token's heads side by
// side) are dispatched together, which keeps HBM accesses row-local.

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

template <int D>
struct GqaGeom {
  static constexpr int kTile = kGqaTileTokens;                 // 32 keys per wave step
  static constexpr int kKB = D / 32;                            // QK k-steps
  static constexpr int kNB = D / 16;                            // PV 16-channel blocks
  static constexpr int kVStride = D + 16;                       // LDS row stride (bf16), breaks bank aliasing
  static constexpr int kVTile = kTile * kVStride;               // bf16 elements per wave
  static constexpr int kChunksPerRow = D / 8;                   // 16-byte chunks per V row
  static constexpr int kVChunks = kTile * kChunksPerRow / 64;   // 16-byte chunks per lane per V tile
  // waves per SIMD the registers are budgeted for: three (twelve streaming
  // waves per CU) is the best measured for the per-request split plan, and
  // the key-range plan launches two; D = 128 fits in 157 VGPRs (168 with a
  // window or packed rows), D = 256 fits two (with a few registers spilled
  // outside the tile loop, reloaded once per piece)
  static constexpr int kWPE = D <= 64 ? 4 : (D <= 128 ? 3 : 2);
  static constexpr int kWPEExt = D <= 64 ? 4 : (D <= 128 ? 3 : 1);   // window / packed rows
};

// Gather one 32-key tile of K or V (linear 16-byte chunks). Keys at or past
// `end` read slots of an already-valid page and are masked later (K) or
// zeroed (V): skipping those loads (exec-masked) measured 5 % slower per
// call. Table entries at or past `end` are never read.
struct TilePages {
  int64_t p0, p1;   // physical pages of keys tok0..tok0+15 and tok0+16..tok0+31
};

// Table entries of the tile at tok0 (tok0 < end), read with scalar loads:
// the table is read-only here, and waiting for a scalar load does not wait
// for the vector-memory K/V loads in flight.
__device__ __forceinline__ TilePages tile_pages(const DecodeGqaArgs &a, const int32_t *bt_row, int tok0, int end) {
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const const_i32 *bt = reinterpret_cast<const const_i32 *>(reinterpret_cast<uintptr_t>(bt_row));
  TilePages tp;
  tp.p0 = bt[tok0 >> a.page_shift];
  tp.p1 = (tok0 + 16 < end) ? (int64_t)bt[(tok0 + 16) >> a.page_shift] : tp.p0;
  return tp;
}

// K rows in the same coalesced pattern as V (16 lanes cover a 256-byte row
// slice): loading straight into the MFMA operand layout would make every
// load instruction touch 16 rows x 64 bytes (half lines), which costs a
// third of the read bandwidth; the operand layout is read back from LDS.
template <int D>
__device__ __forceinline__ void load_k(const DecodeGqaArgs &a, const __bf16 *kbase, const TilePages &tp,
                                       int tok0, int lane, bf16x8 (&k)[GqaGeom<D>::kVChunks]) {
  using G = GqaGeom<D>;
  const int pmask = (1 << a.page_shift) - 1;
#pragma unroll
  for (int c = 0; c < G::kVChunks; ++c) {
    const int idx = c * 64 + lane;
    const int trow = idx / G::kChunksPerRow;
    const int col = (idx % G::kChunksPerRow) * 8;
    const int tok = tok0 + trow;
    const __bf16 *row = kbase + (trow >= 16 ? tp.p1 : tp.p0) * a.k_stride_page + (int64_t)(tok & pmask) * a.k_stride_tok;
    k[c] = load_bf16x8(row + col);   // keys past the end are masked before use
  }
}

template <int D>
__device__ __forceinline__ void load_v(const DecodeGqaArgs &a, const __bf16 *vbase, const TilePages &tp,
                                       int tok0, int end, int lane, bf16x8 (&v)[GqaGeom<D>::kVChunks]) {
  using G = GqaGeom<D>;
  const int pmask = (1 << a.page_shift) - 1;
#pragma unroll
  for (int c = 0; c < G::kVChunks; ++c) {
    const int idx = c * 64 + lane;
    const int trow = idx / G::kChunksPerRow;          // 0..31
    const int col = (idx % G::kChunksPerRow) * 8;
    const int tok = tok0 + trow;
    const __bf16 *row = vbase + (trow >= 16 ? tp.p1 : tp.p0) * a.v_stride_page + (int64_t)(tok & pmask) * a.v_stride_tok;
    const bf16x8 x = load_bf16x8(row + col);
    v[c] = (tok < end) ? x : bf16x8{};
  }
}

// Where a unit's rows live and which keys they see.
struct UnitRows {
  int b, kvh, qg;
  int row;          // this lane's row (lane % 16)
  bool row_valid;
  int64_t ridx;     // this lane's row in [B, q_len, Hq]
  int rr;           // ... and within its request's q_len * Hq rows
  int c0, c1;       // keys of the split any row of the unit sees
  int first;        // first tile of the split the unit walks (tile-aligned, >= c0)
  int begin_max;    // the largest row_begin of the unit's valid rows (wave-uniform)
  int row_begin;    // keys >= row_begin ...
  int row_end;      // ... and < row_end are visible to this lane's row
};

// The unit walks tiles [tile0, tile1) of its request (32-key tiles counted
// from the request's base: 0, or the tile holding its window's first key).
template <bool kExt>
__device__ __forceinline__ UnitRows unit_rows(const DecodeGqaArgs &a, int b, int kvh, int qg, int tile0, int tile1,
                                              int lane) {
  UnitRows u;
  u.b = b;
  u.kvh = kvh;
  u.qg = qg;
  u.row = lane & 15;
  const int lk = a.seq_lens[b];
  int t_row, g_row, t_first, t_last;
  if (kExt && a.packed) {
    // rows t * G + g packed continuously over the q_len tokens ("TokenSpeed-
    // MLA", packed-query paragraph): row r of unit qg is packed row qg*rows + r
    const int total = a.group * a.q_len;
    const int pr = qg * a.rows + u.row;
    u.row_valid = u.row < a.rows && pr < total;
    t_row = u.row_valid ? pr / a.group : 0;
    g_row = u.row_valid ? pr % a.group : 0;
    t_first = (qg * a.rows) / a.group;
    t_last = (min(qg * a.rows + a.rows, total) - 1) / a.group;
  } else {
    // row r of unit qg is query token qg*F + r/G, head kvh*G + r%G
    u.row_valid = u.row < a.rows;
    t_row = qg * a.fold + (u.row_valid ? u.row / a.group : 0);
    g_row = u.row_valid ? u.row % a.group : 0;
    t_first = qg * a.fold;
    t_last = qg * a.fold + a.fold - 1;
  }
  const int h_row = kvh * a.group + g_row;
  int bound = lk, unit_bound = lk;
  if (a.causal) {
    bound = min(lk, max(0, lk - a.q_len + t_row + 1));
    unit_bound = min(lk, max(0, lk - a.q_len + t_last + 1));   // the unit's last token sees most
  }
  // Sliding window ("TokenSpeed-MLA", kernel capability summary, window_left):
  // row t sees no key before lk - q_len - window_left + t. The splits of a
  // request start at its window (tile-aligned), so the walk tracks the window.
  int base = 0, unit_begin = 0;
  u.row_begin = 0;
  if (kExt && a.window_left >= 0) {
    u.row_begin = max(0, lk - a.q_len - a.window_left + t_row);
    unit_begin = max(0, lk - a.q_len - a.window_left + t_first);
    base = max(0, lk - a.q_len - a.window_left) & ~(kGqaTileTokens - 1);
  }
  u.c0 = base + tile0 * kGqaTileTokens;
  u.c1 = min(unit_bound, base + tile1 * kGqaTileTokens);
  u.first = u.c0 + (max(0, unit_begin - u.c0) & ~(kGqaTileTokens - 1));
  u.row_end = min(bound, u.c1);
  u.begin_max = INT32_MIN;   // no row has a lower bound: the mask branch folds away
  if (kExt) {
    int bm = u.row_valid ? u.row_begin : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) bm = max(bm, __shfl_xor(bm, off, 64));
    u.begin_max = __builtin_amdgcn_readfirstlane(bm);
  }
  u.rr = t_row * a.num_q_heads + h_row;
  u.ridx = (int64_t)b * a.q_len * a.num_q_heads + u.rr;
  return u;
}

template <int D>
struct WaveState {
  using G = GqaGeom<D>;
  bf16x8 qop[G::kKB];  // Q^T as the MFMA B operand: row l%16, channels 32kb + 8kg + e
  float m;             // running max, log2 units of the scaled score
  float lsum;          // running sum of bf16-rounded p over this lane's keys
  float lexact;        // running sum of fp32 p over this lane's keys
  f32x4 oacc[G::kNB];  // O^T: lane holds O[row][16nb + 4kg + i]

  __device__ __forceinline__ void init(const DecodeGqaArgs &a, const UnitRows &u, int lane) {
    const int kg = lane >> 4;
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + u.ridx * D;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb) qop[kb] = u.row_valid ? load_bf16x8(qrow + kb * 32 + kg * 8) : bf16x8{};
    m = kNegInf;
    lsum = 0.f;
    lexact = 0.f;
#pragma unroll
    for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Walk tiles first, first + stride, ... below u.c1. Each iteration issues
  // its tile's K and V loads together and then waits for them; nothing is
  // fetched a tile ahead. Measured on the Qwen3-14B-shaped decode: a wave
  // that keeps the next tile's 16 KB in flight while it computes makes the
  // HBM less efficient (more concurrent requests, worse locality) than one
  // whose loads stop while it computes (its neighbours' loads fill the gap):
  // 0.220 vs 0.228 ms per call with twelve waves per CU, and with the key
  // ranges' eight (registers double-buffered, 254 VGPRs, no spills) 0.204
  // vs 0.190 ms.
  __device__ __forceinline__ void walk(const DecodeGqaArgs &a, const UnitRows &u, int first, int stride,
                                       __bf16 *vlds, int lane) {
    const int kg = lane >> 4;
    const int row = lane & 15;
    const int32_t *bt_row = a.block_table + (int64_t)u.b * a.block_table_stride;
    const __bf16 *kbase = static_cast<const __bf16 *>(a.k_cache) + (int64_t)u.kvh * a.k_stride_head;
    const __bf16 *vbase = static_cast<const __bf16 *>(a.v_cache) + (int64_t)u.kvh * a.v_stride_head;
    if (first >= u.c1) return;
    bf16x8 kr[G::kVChunks];
    bf16x8 vr[G::kVChunks];
    for (int tok0 = first; tok0 < u.c1; tok0 += stride) {
      const TilePages tp = tile_pages(a, bt_row, tok0, u.c1);
      load_k<D>(a, kbase, tp, tok0, lane, kr);
      load_v<D>(a, vbase, tp, tok0, u.c1, lane, vr);
      // K tile -> the wave's LDS tile (token-major, padded rows), read back
      // in the MFMA A layout (token = l % 16, 8 channels per lane). LDS
      // operations of one wave execute in order, so the V rows written
      // into the same tile below land after these reads.
#pragma unroll
      for (int c = 0; c < G::kVChunks; ++c) {
        const int idx = c * 64 + lane;
        store_bf16x8_lds(vlds + (idx / G::kChunksPerRow) * G::kVStride + (idx % G::kChunksPerRow) * 8, kr[c]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // S^T tiles: sacc[0] keys tok0 + 4kg + i, sacc[1] keys tok0 + 16 + 4kg + i.
      f32x4 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const __bf16 *krow = vlds + (16 * t + row) * G::kVStride + kg * 8;
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
          sacc[t] = mfma16x16x32(*reinterpret_cast<const bf16x8 *>(krow + kb * 32), qop[kb], sacc[t]);
      }
      // V tile -> the same LDS tile, for the transposing read.
#pragma unroll
      for (int c = 0; c < G::kVChunks; ++c) {
        const int idx = c * 64 + lane;
        store_bf16x8_lds(vlds + (idx / G::kChunksPerRow) * G::kVStride + (idx % G::kChunksPerRow) * 8, vr[c]);
      }
      float x[8];
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = tok0 + 16 * t + 4 * kg + i;
          const float v = (j < u.row_end) ? sacc[t][i] * a.scale_log2 : kNegInf;
          x[4 * t + i] = v;
          mx = fmaxf(mx, v);
        }
      if (tok0 < u.begin_max) {   // the window's lower bound reaches this tile (scalar test)
        mx = kNegInf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = tok0 + 16 * t + 4 * kg + i;
            if (j < u.row_begin) x[4 * t + i] = kNegInf;
            mx = fmaxf(mx, x[4 * t + i]);
          }
      }
      mx = fmaxf(mx, wave_shfl_xor(mx, 16));
      mx = fmaxf(mx, wave_shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      bf16x8 pop;
      float psum = 0.f, pexact = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = exp2_fast(x[e] - m_use);
        const __bf16 pb = to_bf16(pe);
        pop[e] = pb;
        psum += bf16_to_f32(pb);
        pexact += pe;
      }
      lsum = alpha * lsum + psum;
      lexact = alpha * lexact + pexact;
      m = m_new;
#pragma unroll
      for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] *= alpha;
      // LDS writes of this wave must land before its transposing reads.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // O^T[16 channels x 16 rows] += V^T[channels x 32 keys] * P^T[32 keys x rows];
      // k-slot e of lane group kg is key 4kg + e (e < 4) or 16 + 4kg + e - 4.
      const int src_row = 4 * kg + (row >> 2);
      const int src_col = 4 * (row & 3);
#pragma unroll
      for (int nb = 0; nb < G::kNB; ++nb) {
        const bf16x4 lo = lds_read_tr16(vlds + src_row * G::kVStride + nb * 16 + src_col);
        const bf16x4 hi = lds_read_tr16(vlds + (16 + src_row) * G::kVStride + nb * 16 + src_col);
        oacc[nb] = mfma16x16x32(concat(lo, hi), pop, oacc[nb]);
      }
      // The next iteration overwrites this wave's LDS tile: the transposing
      // reads above must have completed first (their results feed the MFMAs,
      // so the compiler waits for them before those issue).
    }
  }

  // Sum the per-lane-group partial sums of each row.
  __device__ __forceinline__ void reduce_sums() {
    lsum += wave_shfl_xor(lsum, 16);
    lsum += wave_shfl_xor(lsum, 32);
    lexact += wave_shfl_xor(lexact, 16);
    lexact += wave_shfl_xor(lexact, 32);
  }
};

// Where a unit's rows go: the final bf16 O and LSE, or FP32 partial rows
// part_base + rr of o_parts / lse_parts.
struct UnitOut {
  bool final_out;
  int64_t part_base;
};

// Rows of an empty unit: LSE -inf; if final also O = 0.
template <int D>
__device__ __forceinline__ void write_empty(const DecodeGqaArgs &a, const UnitRows &u, const UnitOut &out, int lane) {
  if (!u.row_valid) return;
  const int kg = lane >> 4;
  if (out.final_out) {
    __bf16 *dst = static_cast<__bf16 *>(a.o) + u.ridx * D + 4 * kg;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) *reinterpret_cast<u32x2 *>(dst + nb * 16) = u32x2{0u, 0u};
    if (a.lse && kg == 0) a.lse[u.ridx] = kNegInf;
  } else if (kg == 0) {
    a.lse_parts[out.part_base + u.rr] = kNegInf;
  }
}

// One unit: walk tiles [tile0, tile1) of request b for KV head kvh and query
// group qg, and write its rows.
template <int D, bool kExt>
__device__ __forceinline__ void run_unit(const DecodeGqaArgs &a, int b, int kvh, int qg, int tile0, int tile1,
                                         const UnitOut &out, __bf16 *vlds, int lane) {
  using G = GqaGeom<D>;
  const int kg = lane >> 4;
  const UnitRows u = unit_rows<kExt>(a, b, kvh, qg, tile0, tile1, lane);
  if (u.first >= u.c1) {       // no key of this range is visible to the unit
    write_empty<D>(a, u, out, lane);
    return;
  }
  WaveState<D> st;
  st.init(a, u, lane);
  st.walk(a, u, u.first, G::kTile, vlds, lane);
  st.reduce_sums();
  if (!u.row_valid) return;

  // lane holds O[row][16 nb + 4 kg + i]; the rounded-P sum normalises O,
  // the exact sum gives the LSE
  const float inv = (st.lsum > 0.f) ? 1.f / st.lsum : 0.f;
  const float muse = (st.m == kNegInf) ? 0.f : st.m;
  const float lse2 = (st.lexact > 0.f) ? muse + __log2f(st.lexact) : kNegInf;
  if (out.final_out) {
    __bf16 *dst = static_cast<__bf16 *>(a.o) + u.ridx * D + 4 * kg;
#pragma unroll
    for (int nb = 0; nb < G::kNB; ++nb) {
      bf16x4 ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = to_bf16(st.oacc[nb][i] * inv);
      *reinterpret_cast<u32x2 *>(dst + nb * 16) = __builtin_bit_cast(u32x2, ob);
    }
    if (a.lse && kg == 0) a.lse[u.ridx] = lse2;
  } else {
    float *dst = a.o_parts + (out.part_base + u.rr) * D + 4 * kg;
#pragma unroll
    for (int nb = 0; nb < G::kNB; ++nb) *reinterpret_cast<f32x4 *>(dst + nb * 16) = st.oacc[nb] * inv;
    if (kg == 0) a.lse_parts[out.part_base + u.rr] = lse2;
  }
}

// One wave per workgroup. Per-request splits: blockIdx -> (b, split, KV
// head, q group), q group fastest, so the units that read the per-head
// slices of the same token rows are dispatched together; the wave walks its
// split's tiles in order and writes its rows itself (no cross-wave merge,
// a finished wave frees its slot at once).
//
// Key ranges: blockIdx -> (range g, KV head, q group). The tiles of all
// requests, in request order, are cut into ranges of equal length ("Writing
// Page Attention with PyPTO", section 1.3: tasks of equal size keep every
// core busy to the end), so every wave of the launch streams the same
// number of bytes and the launch ends when its waves do, not when its
// longest requests do. A range that crosses request boundaries walks one
// piece per request; a request that lies inside one range is written
// final, the others as partial rows g + b that the merge combines. All
// waves of a range read the same token rows at the same time.
//
// kExt adds what a sliding window or packed query rows need (the
// lower-bound mask, the packed row mapping); it is a separate instantiation
// so the plain kernel keeps its registers (at D = 256 it also runs at a
// lower occupancy than the plain one).
template <int D, bool kExt>
__global__ __launch_bounds__(64, kExt ? GqaGeom<D>::kWPEExt : GqaGeom<D>::kWPE) void decode_gqa_wave_kernel(const DecodeGqaArgs a) {
  using G = GqaGeom<D>;
  __shared__ __attribute__((aligned(16))) __bf16 vlds[G::kVTile];
  const int lane = threadIdx.x;
  int unit = blockIdx.x;
  const int qg = unit % a.q_groups;
  unit /= a.q_groups;
  const int kvh = unit % a.num_kv_heads;
  unit /= a.num_kv_heads;
  // The wave walks pieces (b, [s0, s1)) of the tiles [t_lo, t_hi): with
  // splits one piece, tiles [split L, split L + L) of request b; with key
  // ranges every request its range meets.
  const int wl = kExt ? a.window_left : -1;
  const int64_t rows_req = (int64_t)a.q_len * a.num_q_heads;
  const bool ranges_mode = a.key_ranges > 0;
  int g = 0, split = 0, b = 0, p = 0, t_lo, t_hi;
  if (!ranges_mode) {
    split = unit % a.num_splits;
    b = unit / a.num_splits;
    const int st = a.split_tokens / kGqaTileTokens;
    t_lo = split * st;
    t_hi = t_lo + st;
  } else {
    g = unit;
    const BatchTiles bt = batch_tiles(a.seq_lens, a.batch, a.q_len, wl, 0, lane);
    const int total = __builtin_amdgcn_readfirstlane(bt.total);
    const int ranges = min(a.key_ranges, total);
    if (g >= ranges) return;
    t_lo = key_range_start(g, ranges, total);
    t_hi = key_range_start(g + 1, ranges, total);
    // the request holding tile t_lo, and its first tile
    int carry = 0;
#pragma unroll
    for (int k = 0; k < kKeyRangeMaxBatch / 64; ++k) {
      int incl = bt.n[k];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int up = __shfl_up(incl, off, 64);
        incl += (lane >= off) ? up : 0;
      }
      incl += carry;
      const uint64_t hit = __ballot(incl > t_lo && lane + 64 * k < a.batch);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        b = 64 * k + l;
        p = __shfl(incl - bt.n[k], l, 64);
        break;
      }
      carry = __shfl(incl, 63, 64);
    }
    b = __builtin_amdgcn_readfirstlane(b);
    p = __builtin_amdgcn_readfirstlane(p);
  }
  while (p < t_hi) {
    const int n = ranges_mode ? gqa_request_tiles(a.seq_lens[b], a.q_len, wl) : t_hi;
    const int s0 = max(t_lo, p) - p, s1 = min(t_hi, p + n) - p;
    const UnitOut out = ranges_mode ? UnitOut{s0 == 0 && s1 == n, (int64_t)(g + b) * rows_req}
                                    : UnitOut{a.num_splits == 1, ((int64_t)split * a.batch + b) * rows_req};
    run_unit<D, kExt>(a, b, kvh, qg, s0, s1, out, vlds, lane);
    p += n;
    ++b;
  }
}

template <int D>
hipError_t launch_d(const DecodeGqaArgs &a, hipStream_t stream) {
  const int64_t units = (int64_t)(a.key_ranges > 0 ? a.key_ranges : a.batch * a.num_splits) * a.num_kv_heads * a.q_groups;
  if (a.packed || a.window_left >= 0)
    hipLaunchKernelGGL((decode_gqa_wave_kernel<D, true>), dim3((unsigned)units), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_gqa_wave_kernel<D, false>), dim3((unsigned)units), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int decode_gqa_waves_per_cu(int head_dim, bool ext) {
  switch (head_dim) {
    case 64: return 4 * (ext ? GqaGeom<64>::kWPEExt : GqaGeom<64>::kWPE);
    case 128: return 4 * (ext ? GqaGeom<128>::kWPEExt : GqaGeom<128>::kWPE);
    default: return 4 * (ext ? GqaGeom<256>::kWPEExt : GqaGeom<256>::kWPE);
  }
}

hipError_t launch_decode_gqa(const DecodeGqaArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    case 256: return launch_d<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
