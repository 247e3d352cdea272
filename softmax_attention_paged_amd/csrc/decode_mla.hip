// MLA-shaped paged decode over one latent KV head, split over the KV sequence,
// for gfx950.
//
// The cache row of a token is the 576-wide latent: K is the whole row and V
// its first 512 entries ("TokenSpeed-MLA", kernel capability summary: query
// width kv_lora_rank + qk_rope_head_dim; a [num_pages, page_size, D_total]
// cache). The query heads and F folded query tokens form up to 128 MFMA rows
// ("TokenSpeed-MLA", section "Key Optimization ... Group q_seqlen and
// num_heads into BMM1 M": with 64 heads and 4 tokens, F = 2 gives 128 rows
// and two query groups). Each workgroup is one (request, query group, KV
// split) and writes split partials merged by log-sum-exp in a second kernel
// ("TokenSpeed-MLA", section "Decode performance").
//
// Workgroup: 4 waves x 32 rows at one wave per SIMD, so that the 32 x 512
// FP32 output block of a wave (256 registers per lane) fills the accumulation
// registers; the query operand of the first 256 columns stays in vector
// registers, the other 320 columns wait in LDS (rows padded to 656 bytes,
// bank-conflict-free; 84 KB, with the two 36 KB tiles 156 KB of the CU's
// 160 KB). Per 32-key tile:
//   - the latent tile is gathered through the block table ONCE into LDS
//     (double-buffered, one tile ahead): bf16 rows by direct HBM -> LDS
//     loads, fp8 e4m3 rows through registers, widened to bf16 exactly on the
//     way (every e4m3 value is a bf16 value), the per-tensor scale applied to
//     the scores and the final output instead ("TokenSpeed-MLA": FP8 KV with
//     FP32 softmax exponentials and sums, bf16 output). The same LDS bytes
//     serve as K and, for the first 512 columns, as V;
//   - S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16: each K or V
//     operand read from LDS feeds 32 rows; the row state is lane-local and P
//     is the B operand straight from the score registers; V^T is read with
//     ds_read_b64_tr_b16;
//   - static-anchor softmax ("Flywheel Attention", section "Static-anchor
//     softmax" and Appendix A): each row fixes its anchor at the max of the
//     scores it may see in the first walked tile that holds one, with every
//     mask applied first (so the anchor is one of the row's own scores and
//     its sum is at least 1), and never moves it, so O is never rescaled (it
//     stays in the accumulation registers, untouched by vector ALU work);
//     after each tile the running sum is checked against 2^kAnchorLog2, which
//     bounds every exponential taken so far. A failed check (a score far
//     above the anchor, or an overflow) makes the whole workgroup walk its
//     split again with the failing rows' anchors raised to that tile's max;
//     after a second failure, one walk raises every anchor to its row's max
//     over the split and the last walk, in which no exponential exceeds 1,
//     runs unchecked. The pages replay one block from saved state instead,
//     which would need a second copy of O. One FP32 sum of the exponentials
//     normalises O and gives the LSE.
// Workgroups are renumbered so that consecutive units run on the same XCD:
// the query groups of one split then share that XCD's L2 for the latent.

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kW = 4;                              // waves, 32 rows each
constexpr int kThreads = 64 * kW;
constexpr int kTileN = kMlaTileTokens;             // 32 keys per tile
constexpr int kRowB = kDk * 2;                     // bytes of a latent row in LDS
constexpr int kChunks = kDk / 8;                   // 16-byte chunks per row
constexpr int kTileB = kTileN * kRowB;             // bytes of one LDS tile
constexpr int kKB = kDk / 16;                      // 36 QK k-steps
constexpr int kKBReg = 16;                         // k-steps whose Q operand stays in registers
constexpr int kRing = 3;                           // LDS operand reads in flight ahead of the MFMAs
constexpr int kQRowB = (kDk - 16 * kKBReg) * 2 + 16;   // LDS bytes per row of the other Q columns (padded)
constexpr int kNB = kDv / 32;                      // 16 PV channel blocks
constexpr int kDma = kTileN * kChunks / 64 / kW;   // 9 direct loads per wave per bf16 tile
constexpr int kF8Chunks = kTileN * (kDk / 16);     // 16-byte fp8 chunks per tile
constexpr int kF8PerThread = (kF8Chunks + kThreads - 1) / kThreads;
constexpr int kXcds = 8;
// A row's running sum may reach 2^kAnchorLog2 before its split restarts: then
// every exponential is at most 2^40, a split's sum at most 2^60 (splits hold
// under 2^20 keys), and O at most |V|max 2^60 (finite for fp8 codes, |c| <=
// 448, and for bf16 latents below 2^67).
constexpr float kAnchorLog2 = 40.0f;
static_assert(kTileN * kChunks % (64 * kW) == 0, "whole direct loads per tile");
static_assert(kW * 32 == kMlaRows, "rows per workgroup");

// LDS rows are unpadded; 16-byte chunk c of row r sits at slot c ^ swz(r).
// With the 1152-byte row stride (rows alternate bank halves) this keeps the
// 16 rows of a K-operand read and the 4 rows x 4 chunks of a transposing V
// read on distinct banks. swz < 8, so a chunk stays in its aligned group of 8.
__device__ __forceinline__ int mla_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Bijective renumbering: hardware dispatches workgroup i to XCD i % 8; unit
// numbers handed to one XCD become consecutive.
__device__ __forceinline__ int xcd_unit(int i, int n) {
  const int per = n / kXcds, rem = n % kXcds;
  const int x = i % kXcds, k = i / kXcds;
  return x * per + min(x, rem) + k;
}

// Where this thread's tile loads go. bf16: load k of the wave fills LDS slot
// (k kW + wave) 64 + lane; fp8: chunk c of the thread is fp8 chunk
// c kThreads + tid of the tile (row, 16 codes).
struct MlaLoadMap {
  uint32_t off[kDma > kF8PerThread ? kDma : kF8PerThread];   // byte offset from the tile's first row
};

template <bool FP8>
__device__ __forceinline__ void mla_row_chunk(int c, int wave, int lane, int tid, int &row, int &chunk) {
  if constexpr (FP8) {
    const int idx = c * kThreads + tid;
    row = idx / (kDk / 16);
    chunk = idx % (kDk / 16);
  } else {
    const int slot = (c * kW + wave) * 64 + lane;
    row = slot / kChunks;
    chunk = (slot % kChunks) ^ mla_swz(row);   // global chunk stored at this slot
  }
}

struct MlaCtx {
  const char *kv;          // cache bytes
  int64_t page_b, tok_b;   // page / token strides in bytes
  const int32_t *bt_row;
  int page_shift, pmask;
  bool wide;               // every tile lies inside one page
};

// Issue the loads of the tile at key j0 (keys >= end are zero). bf16: direct
// HBM -> LDS into `dst`; fp8: into the thread's stage registers.
template <bool FP8>
__device__ __forceinline__ void mla_issue(const MlaCtx &x, const MlaLoadMap &map, int j0, int end, int wave, int lane,
                                          int tid, char *dst, u32x4 (&stage)[kF8PerThread]) {
  if (x.wide && j0 + kTileN <= end) {
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const int64_t page = reinterpret_cast<const_i32 *>(reinterpret_cast<uintptr_t>(x.bt_row))[j0 >> x.page_shift];
    const char *tile = x.kv + page * x.page_b + (int64_t)(j0 & x.pmask) * x.tok_b;
    if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < kF8PerThread; ++c)
        stage[c] = (c * kThreads + tid < kF8Chunks) ? *reinterpret_cast<const u32x4 *>(tile + map.off[c])
                                                    : u32x4{0u, 0u, 0u, 0u};
    } else {
      const uint32_t lds = lds_address(dst);
#pragma unroll
      for (int k = 0; k < kDma; ++k) lds_dma16(tile, map.off[k], lds + (k * kW + wave) * 1024);
    }
    return;
  }
  // row by row: the tail tile, or pages smaller than a tile
  constexpr int kN = FP8 ? kF8PerThread : kDma;
#pragma unroll
  for (int c = 0; c < kN; ++c) {
    int row, chunk;
    mla_row_chunk<FP8>(c, wave, lane, tid, row, chunk);
    const int j = j0 + row;
    const bool in = (!FP8 || c * kThreads + tid < kF8Chunks) && j < end;
    const char *src = nullptr;
    if (in) {
      const int64_t page = x.bt_row[j >> x.page_shift];
      src = x.kv + page * x.page_b + (int64_t)(j & x.pmask) * x.tok_b + chunk * 16;
    }
    if constexpr (FP8) {
      stage[c] = in ? *reinterpret_cast<const u32x4 *>(src) : u32x4{0u, 0u, 0u, 0u};
    } else {
      const int slot = (c * kW + wave) * 64 + lane;
      if (in)
        lds_dma16(src, lds_address(dst + slot * 16));
      else
        *reinterpret_cast<u32x4 *>(dst + slot * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Pull the cache lines of the whole tile at key j0 (inside one page) into
// L2 ahead of its loads: one dword per 128-byte line of each row, loaded
// straight into a scratch LDS word of the lane (`sink`: the wave's 256 bytes,
// never read), so no register waits for it. The tile's own loads, issued an
// iteration later, then hit in L2 instead of waiting out an HBM round trip
// with only one tile in flight per CU.
template <bool FP8>
__device__ __forceinline__ void mla_prefetch(const MlaCtx &x, int j0, int tid, uint32_t sink) {
  constexpr int kLines = (kDk * (FP8 ? 1 : 2) + 127) / 128;   // 128-byte lines a row spans
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const int64_t page = reinterpret_cast<const_i32 *>(reinterpret_cast<uintptr_t>(x.bt_row))[j0 >> x.page_shift];
  const char *tile = x.kv + page * x.page_b + (int64_t)(j0 & x.pmask) * x.tok_b;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + k * kThreads;
    if (i < kTileN * kLines) {
      const uint32_t off = static_cast<uint32_t>((i / kLines) * x.tok_b + (i % kLines) * 128);
      asm volatile("global_load_lds_dword %0, %1" : : "v"(off), "s"(tile), "{m0}"(sink) : "memory");
    }
  }
}

// fp8: widen the staged codes and store them as bf16 rows.
__device__ __forceinline__ void mla_store_fp8(char *dst, int tid, const u32x4 (&stage)[kF8PerThread]) {
#pragma unroll
  for (int c = 0; c < kF8PerThread; ++c) {
    const int idx = c * kThreads + tid;
    if (idx >= kF8Chunks) continue;
    const int row = idx / (kDk / 16), c8 = idx % (kDk / 16);
    bf16x8 lo, hi;
    fp8x16_to_bf16(stage[c], lo, hi);
    char *r = dst + row * kRowB;
    store_bf16x8_lds(r + ((2 * c8) ^ mla_swz(row)) * 16, lo);
    store_bf16x8_lds(r + ((2 * c8 + 1) ^ mla_swz(row)) * 16, hi);
  }
}

// FP8 q: the codes also stay in LDS as the K operand of the FP8 matrix
// instruction (576-byte rows; the 16-byte chunks of row r XOR-swizzled by
// (r >> 2) & 3, which puts rows r, r + 4, r + 8, r + 12 of an operand read
// on different banks and keeps each chunk in its aligned group of four),
// and only the 512 V columns are widened to the bf16 tile.
constexpr int kK8RowB = kDk;                         // bytes of a code row
constexpr int kK8TileB = kTileN * kK8RowB;           // bytes of a code tile
constexpr int kKB8 = kDk / 64;                       // FP8 QK k-steps of 64 codes
constexpr int kKB8Reg = 6;                           // k-steps whose q codes stay in registers
constexpr int kQ8RowB = (kKB8 - kKB8Reg) * 64 + 16;  // LDS bytes per row of the other q codes (padded)
__device__ __forceinline__ int k8_swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void mla_store_fp8q(char *vdst, char *kdst, int tid, const u32x4 (&stage)[kF8PerThread]) {
#pragma unroll
  for (int c = 0; c < kF8PerThread; ++c) {
    const int idx = c * kThreads + tid;
    if (idx >= kF8Chunks) continue;
    const int row = idx / (kDk / 16), c8 = idx % (kDk / 16);
    *reinterpret_cast<u32x4 *>(kdst + row * kK8RowB + (c8 ^ k8_swz(row)) * 16) = stage[c];
    if (c8 < kDv / 16) {
      bf16x8 lo, hi;
      fp8x16_to_bf16(stage[c], lo, hi);
      char *r = vdst + row * kRowB;
      store_bf16x8_lds(r + ((2 * c8) ^ mla_swz(row)) * 16, lo);
      store_bf16x8_lds(r + ((2 * c8 + 1) ^ mla_swz(row)) * 16, hi);
    }
  }
}

typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // format selectors 0, 0: both operands E4M3; zero scale operands give the
  // unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  i32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = static_cast<int>(lo[i]);
    r[4 + i] = static_cast<int>(hi[i]);
  }
  return r;
}

// kExt adds what a sliding window or packed query rows need (the packed row
// mapping, the window's start and lower-bound mask); the plain kernel keeps
// those registers free. QF8 (with FP8): E4M3 q, QK on the FP8 instruction.
template <bool FP8, bool QF8, bool kExt>
__global__ __launch_bounds__(kThreads, 1) void decode_mla_kernel(const DecodeMlaArgs a) {
  static_assert(!QF8 || FP8, "fp8 q comes with an fp8 cache");
  __shared__ __attribute__((aligned(16))) char tiles[2 * kTileB];
  __shared__ __attribute__((aligned(16))) char qlds[QF8 ? kMlaRows * kQ8RowB : kMlaRows * kQRowB];
  __shared__ __attribute__((aligned(16))) char ktiles8[QF8 ? 2 * kK8TileB : 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int r32 = lane & 31;

  const int n_units = a.batch * a.num_splits * a.q_groups;
  int unit = xcd_unit(blockIdx.x, n_units);
  const int qg = unit % a.q_groups;
  unit /= a.q_groups;
  const int split = unit % a.num_splits;
  const int b = unit / a.num_splits;

  const int lk = a.seq_lens[b];
  // this lane's row r = 32 * wave + lane % 32: folded, query token qg*F + r/H
  // and head r%H; packed ("TokenSpeed-MLA", packed-query paragraph), packed
  // row qg*rows + r = token * H + head
  const int r = 32 * wave + r32;
  int t_row, h_row, t_first, t_last;
  bool row_valid;
  if (kExt && a.packed) {
    const int total = a.num_heads * a.q_len;
    const int pr = qg * a.rows + r;
    row_valid = r < a.rows && pr < total;
    t_row = row_valid ? pr / a.num_heads : 0;
    h_row = row_valid ? pr % a.num_heads : 0;
    t_first = (qg * a.rows) / a.num_heads;
    t_last = (min(qg * a.rows + a.rows, total) - 1) / a.num_heads;
  } else {
    row_valid = r < a.rows;
    t_row = qg * a.fold + (row_valid ? r / a.num_heads : 0);
    h_row = row_valid ? r % a.num_heads : 0;
    t_first = qg * a.fold;
    t_last = qg * a.fold + a.fold - 1;
  }
  int unit_bound = lk, bound = lk;
  if (a.causal) {
    unit_bound = min(lk, max(0, lk - a.q_len + t_last + 1));
    bound = min(lk, max(0, lk - a.q_len + t_row + 1));
  }
  // Sliding window ("TokenSpeed-MLA", kernel capability summary, window_left):
  // row t sees no key before lk - q_len - window_left + t; a request's splits
  // start at its window (tile-aligned), so the walk tracks the window.
  int base = 0, unit_begin = 0, row_begin = 0;
  if (kExt && a.window_left >= 0) {
    row_begin = max(0, lk - a.q_len - a.window_left + t_row);
    unit_begin = max(0, lk - a.q_len - a.window_left + t_first);
    base = max(0, lk - a.q_len - a.window_left) & ~(kTileN - 1);
  }
  // wave-uniform by construction; said explicitly so the tile addresses
  // derived from them stay in scalar registers
  const int c0 = __builtin_amdgcn_readfirstlane(base + split * a.split_tokens);
  const int c1 = __builtin_amdgcn_readfirstlane(min(unit_bound, c0 + a.split_tokens));
  const int first = __builtin_amdgcn_readfirstlane(c0 + (max(0, unit_begin - c0) & ~(kTileN - 1)));
  const int64_t R = (int64_t)a.batch * a.q_len * a.num_heads;
  const int64_t ridx = ((int64_t)b * a.q_len + t_row) * a.num_heads + h_row;
  const int row_end = min(bound, c1);

  if (first >= c1) {   // uniform: no key of this split is visible
    if (row_valid) {
      if (a.num_splits == 1) {
        __bf16 *dst = static_cast<__bf16 *>(a.o) + ridx * kDv + 4 * half;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) *reinterpret_cast<u32x2 *>(dst + 32 * nb + 8 * g) = u32x2{0u, 0u};
        if (a.lse && half == 0) a.lse[ridx] = kNegInf;
      } else if (half == 0) {
        a.lse_parts[(int64_t)split * R + ridx] = kNegInf;
      }
    }
    return;
  }

  // keys some valid row of this wave must mask: from valid_min up, and below
  // begin_max (scalars, so the per-tile tests are branches)
  int valid_min = row_valid ? row_end : 0x7fffffff;
  int begin_max = (kExt && row_valid) ? row_begin : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    valid_min = min(valid_min, __shfl_xor(valid_min, off, 64));
    begin_max = max(begin_max, __shfl_xor(begin_max, off, 64));
  }
  valid_min = __builtin_amdgcn_readfirstlane(valid_min);
  begin_max = __builtin_amdgcn_readfirstlane(begin_max);
  const bool wave_active = 32 * wave < a.rows;

  // Q^T operand: lane holds Q[row r][16 kb + 8 half .. +8]; a negative scale
  // negates Q (exact in bf16) so that c > 0
  const float c = fabsf(a.scale_log2);
  const u32x4 qsign = (a.scale_log2 < 0.f) ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u} : u32x4{};
  bf16x8 qop[kKBReg];
  // FP8 q: codes 64 kb + 32 half .. + 31 of row r; k-steps past kKB8Reg
  // wait in the row's LDS copy
  i32x8 qop8[QF8 ? kKB8Reg : 1];
  if constexpr (QF8) {
    const unsigned s8 = (a.scale_log2 < 0.f) ? 0x80808080u : 0u;   // a sign flip of every code is exact
    const u32x4 sg = u32x4{s8, s8, s8, s8};
    const uint8_t *qrow = static_cast<const uint8_t *>(a.q) + ridx * kDk;
    char *qdst = qlds + r * kQ8RowB;
#pragma unroll
    for (int kb = 0; kb < kKB8; ++kb) {
      u32x4 lo = u32x4{0u, 0u, 0u, 0u}, hi = lo;
      if (row_valid) {
        lo = *reinterpret_cast<const u32x4 *>(qrow + 64 * kb + 32 * half) ^ sg;
        hi = *reinterpret_cast<const u32x4 *>(qrow + 64 * kb + 32 * half + 16) ^ sg;
      }
      if (kb < kKB8Reg) {
        qop8[kb < kKB8Reg ? kb : 0] = cat8(lo, hi);
      } else {
        *reinterpret_cast<u32x4 *>(qdst + (kb - kKB8Reg) * 64 + 32 * half) = lo;
        *reinterpret_cast<u32x4 *>(qdst + (kb - kKB8Reg) * 64 + 32 * half + 16) = hi;
      }
    }
  } else {
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + ridx * kDk;
#pragma unroll
    for (int kb = 0; kb < kKBReg; ++kb)
      qop[kb] = row_valid ? __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, load_bf16x8(qrow + kb * 16 + half * 8)) ^ qsign)
                          : bf16x8{};
    // the other columns: chunk 2 (kb - kKBReg) + half of the row's LDS copy
    char *qdst = qlds + r * kQRowB;
#pragma unroll
    for (int kb = kKBReg; kb < kKB; ++kb) {
      const u32x4 v = row_valid ? __builtin_bit_cast(u32x4, load_bf16x8(qrow + kb * 16 + half * 8)) ^ qsign : u32x4{};
      *reinterpret_cast<u32x4 *>(qdst + (2 * (kb - kKBReg) + half) * 16) = v;
    }
  }
  const char *qsrc = qlds + r * kQRowB + half * 16;

  // LDS operand offsets: chunk 2 kb + half of key row r32 is at
  // koff[kb % 4] + 128 (kb / 4); the V^T reads (see the prefill kernel for the
  // lane mapping) at voff[lo/hi][nb % 2] + 128 (nb / 2) + 16 kk rows
  int koff[4];
  {
    const int f = mla_swz(r32);
#pragma unroll
    for (int t = 0; t < 4; ++t) koff[t] = r32 * kRowB + ((2 * t + half) ^ f) * 16;
  }
  int voff[2][2];
  {
    const int s16 = lane & 15;
    const int row0 = 4 * half + (s16 >> 2);
    const int cb = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
    const int f0 = mla_swz(row0), f1 = mla_swz(row0 + 8);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      voff[0][q] = row0 * kRowB + ((4 * q + cb) ^ f0) * 16 + 8 * (s16 & 1);
      voff[1][q] = (row0 + 8) * kRowB + ((4 * q + cb) ^ f1) * 16 + 8 * (s16 & 1);
    }
  }

  MlaCtx x;
  x.kv = static_cast<const char *>(a.kv_cache);
  x.page_b = a.kv_stride_page * (FP8 ? 1 : 2);
  x.tok_b = a.kv_stride_tok * (FP8 ? 1 : 2);
  x.bt_row = a.block_table + (int64_t)b * a.block_table_stride;
  x.page_shift = a.page_shift;
  x.pmask = (1 << a.page_shift) - 1;
  x.wide = (1 << a.page_shift) >= kTileN;   // tiles start at multiples of 32 keys
  MlaLoadMap map;
#pragma unroll
  for (int k = 0; k < (FP8 ? kF8PerThread : kDma); ++k) {
    int row, chunk;
    mla_row_chunk<FP8>(k, wave, lane, tid, row, chunk);
    map.off[k] = static_cast<uint32_t>(row * x.tok_b + chunk * 16);
  }

  __shared__ int restart;                     // set by a wave whose rows failed the anchor check
  if (tid == 0) restart = 0;
  float anchor = kNegInf;                     // this row's static anchor (log2 units); -inf: no key yet
  float lsum = 0.f;
  f32x16 oacc[kNB];
  const int ntiles = (c1 - first + kTileN - 1) / kTileN;
  u32x4 stage[kF8PerThread];
  __shared__ __attribute__((aligned(16))) char sink_lds[kW * 256];   // prefetch destinations, never read
  const uint32_t sink = lds_address(sink_lds + wave * 256);
  const float sum_limit = exp2f(kAnchorLog2);

  // Walks: 0 checked; 1 checked, with the anchors 0 raised; on a second
  // failure 2 rises (each anchor becomes its row's max over the split, the
  // walk's O is dropped) and 3 runs unchecked, since no exponential exceeds 1
  // (a split's sum is at most its 2^20 keys).
  bool rising = false;
  for (int attempt = 0;; ++attempt) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) oacc[nb] = f32x16{};
    lsum = 0.f;
    mla_issue<FP8>(x, map, first, c1, wave, lane, tid, tiles, stage);
    if (x.wide && first + 2 * kTileN <= c1) mla_prefetch<FP8>(x, first + kTileN, tid, sink);
    if constexpr (QF8) mla_store_fp8q(tiles, ktiles8, tid, stage);
    else if constexpr (FP8) mla_store_fp8(tiles, tid, stage);
    for (int it = 0; it < ntiles; ++it) {
      const int j0 = first + it * kTileN;
      const int p = it & 1;
      // tile it has landed for every wave; every wave is done with tile it-1,
      // whose buffer takes tile it+1 (whose lines the previous iteration
      // pulled into L2); the lines of tile it+2 are prefetched next
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (restart) break;                     // uniform: read after the barrier
      if (it + 1 < ntiles) mla_issue<FP8>(x, map, j0 + kTileN, c1, wave, lane, tid, tiles + (p ^ 1) * kTileB, stage);
      if (x.wide && j0 + 3 * kTileN <= c1) mla_prefetch<FP8>(x, j0 + 2 * kTileN, tid, sink);

      if (wave_active) {
        const char *tile = tiles + p * kTileB;
        // S^T: lane holds keys j0 + 8(i/4) + 4 half + i%4 of row r32
        // Operands come from LDS kRing MFMAs ahead of use (one wave per SIMD:
        // no other wave hides the LDS latency); the fences keep that order.
        f32x16 s = f32x16{};
        if constexpr (QF8) {
          // 9 FP8 k-steps of 64 codes: chunks 4 kb + 2 half (+1) of key row r32
          const char *krow = ktiles8 + p * kK8TileB + r32 * kK8RowB;
          const int sw = k8_swz(r32);
          auto kread8 = [&](int kb) {
            return cat8(*reinterpret_cast<const u32x4 *>(krow + ((4 * kb + 2 * half) ^ sw) * 16),
                        *reinterpret_cast<const u32x4 *>(krow + ((4 * kb + 2 * half + 1) ^ sw) * 16));
          };
          const char *q8src = qlds + r * kQ8RowB + 32 * half;
          auto qread8 = [&](int kb) {
            return (kb < kKB8Reg) ? qop8[kb < kKB8Reg ? kb : 0]
                                  : cat8(*reinterpret_cast<const u32x4 *>(q8src + (kb - kKB8Reg) * 64),
                                         *reinterpret_cast<const u32x4 *>(q8src + (kb - kKB8Reg) * 64 + 16));
          };
          i32x8 kr8[kRing], qr8[kRing];
#pragma unroll
          for (int i = 0; i < kRing; ++i) {
            kr8[i] = kread8(i);
            qr8[i] = qread8(i);
          }
#pragma unroll
          for (int kb = 0; kb < kKB8; ++kb) {
            __builtin_amdgcn_sched_barrier(0);
            s = mfma_f8(kr8[kb % kRing], qr8[kb % kRing], s);
            if (kb + kRing < kKB8) {
              kr8[kb % kRing] = kread8(kb + kRing);
              qr8[kb % kRing] = qread8(kb + kRing);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
          auto kread = [&](int kb) { return *reinterpret_cast<const bf16x8 *>(tile + koff[kb & 3] + (kb >> 2) * 128); };
          auto qread = [&](int kb) {
            return (kb < kKBReg) ? qop[kb < kKBReg ? kb : 0]
                                 : *reinterpret_cast<const bf16x8 *>(qsrc + (kb - kKBReg) * 32);
          };
          bf16x8 kr[kRing], qr[kRing];
#pragma unroll
          for (int i = 0; i < kRing; ++i) {
            kr[i] = kread(i);
            qr[i] = qread(i);
          }
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb) {
            __builtin_amdgcn_sched_barrier(0);
            s = mfma32x32x16(kr[kb % kRing], qr[kb % kRing], s);
            if (kb + kRing < kKB) {
              kr[kb % kRing] = kread(kb + kRing);
              qr[kb % kRing] = qread(kb + kRing);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (j0 + kTileN > valid_min) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = j0 + 8 * (i >> 2) + 4 * half + (i & 3);
            s[i] = (j < row_end) ? s[i] : kNegInf;
          }
        }
        if (kExt && j0 < begin_max) {         // the window's lower bound (scalar test)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = j0 + 8 * (i >> 2) + 4 * half + (i & 3);
            s[i] = (j >= row_begin) ? s[i] : kNegInf;
          }
        }
        // The anchor: the max of the scores the row may see, in the first
        // tile of the walk that holds one. The masks above come first, so a
        // key hidden by the window or the causal bound never sets it. In the
        // first walk a row's first visible key lies in its first two tiles
        // (the walk starts at the tile of the unit's first row's first key,
        // and the rows of a unit start at most q_len - 1 <= 3 keys apart); a
        // restarted walk also sets the anchors its abandoned predecessor did
        // not reach. A rising walk takes every tile's max (its O is dropped).
        if (it < 2 || attempt > 0) {          // uniform: later tiles of the first walk skip it
          float mx = kNegInf;
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
          const float mt = half_max(mx) * c;
          if (it == 0 && attempt == 0) anchor = mt;
          if (it == 1 || attempt > 0) anchor = (anchor == kNegInf) ? mt : anchor;
          anchor = rising ? fmaxf(anchor, mt) : anchor;
        }
        const float a_use = (anchor == kNegInf) ? 0.f : anchor;
        bf16x8 pop[2];
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pe = exp2_fast(__builtin_fmaf(s[i], c, -a_use));
          pop[i >> 3][i & 7] = to_bf16(pe);
          if (i & 1) ps1 += pe; else ps0 += pe;
        }
        lsum += half_sum(ps0 + ps1);
        if (attempt < 2 && __ballot(!(lsum <= sum_limit) && lsum == lsum)) {
          // some row's sum left the budget (NaN sums, from NaN inputs, pass
          // through): raise those rows' anchors to this tile's max and start over
          float mx = kNegInf;
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
          const float mt = half_max(mx) * c;
          if (!(lsum <= sum_limit)) anchor = fmaxf(anchor, mt);
          restart = 1;
        }
        // O^T += V^T P^T; V is the first 512 columns of the latent tile
        {
          // step t: k-step t / kNB (16 keys), channel block t % kNB
          auto vread = [&](int t) {
            const char *vb = tile + (t / kNB) * 16 * kRowB + ((t % kNB) >> 1) * 128;
            return concat(lds_read_tr16(vb + voff[0][t & 1]), lds_read_tr16(vb + voff[1][t & 1]));
          };
          bf16x8 vr[kRing];
#pragma unroll
          for (int i = 0; i < kRing; ++i) vr[i] = vread(i);
#pragma unroll
          for (int t = 0; t < 2 * kNB; ++t) {
            __builtin_amdgcn_sched_barrier(0);
            oacc[t % kNB] = mfma32x32x16(vr[t % kRing], pop[t / kNB], oacc[t % kNB]);
            if (t + kRing < 2 * kNB) vr[t % kRing] = vread(t + kRing);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (QF8) {
        if (it + 1 < ntiles) mla_store_fp8q(tiles + (p ^ 1) * kTileB, ktiles8 + (p ^ 1) * kK8TileB, tid, stage);
      } else if constexpr (FP8) {
        if (it + 1 < ntiles) mla_store_fp8(tiles + (p ^ 1) * kTileB, tid, stage);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int again = restart;
    __syncthreads();                          // every wave has read the flag before it is cleared
    if (attempt == 2) {                       // the rising walk: every anchor is now its row's max
      rising = false;
      continue;
    }
    if (!again || attempt == 3) break;
    if (tid == 0) restart = 0;
    rising = attempt == 1;                    // second failure
  }

  // ---- epilogue: each wave writes its own rows ----
  const float l = lsum;                        // already summed over the two halves
  if (!row_valid) return;
  const float inv = (l > 0.f) ? a.kv_scale / l : 0.f;     // V dequantisation folded in
  const float muse = (anchor == kNegInf) ? 0.f : anchor;
  const float lse2 = (l > 0.f) ? muse + __log2f(l) : kNegInf;
  if (a.num_splits == 1) {
    __bf16 *dst = static_cast<__bf16 *>(a.o) + ridx * kDv + 4 * half;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ob;
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i] = to_bf16(oacc[nb][4 * g + i] * inv);
        *reinterpret_cast<u32x2 *>(dst + 32 * nb + 8 * g) = __builtin_bit_cast(u32x2, ob);
      }
    if (a.lse && half == 0) a.lse[ridx] = lse2;
  } else {
    float *dst = a.o_parts + ((int64_t)split * R + ridx) * kDv + 4 * half;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = oacc[nb][4 * g + i] * inv;
        *reinterpret_cast<f32x4 *>(dst + 32 * nb + 8 * g) = ov;
      }
    if (half == 0) a.lse_parts[(int64_t)split * R + ridx] = lse2;
  }
}

}  // namespace

hipError_t launch_decode_mla(const DecodeMlaArgs &a, hipStream_t stream) {
  const int64_t units = (int64_t)a.batch * a.num_splits * a.q_groups;
  const bool ext = a.packed || a.window_left >= 0;
  const dim3 grid((unsigned)units), block(kThreads);
  if (a.kv_fp8 && a.q_fp8) {
    if (ext) hipLaunchKernelGGL((decode_mla_kernel<true, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_mla_kernel<true, true, false>), grid, block, 0, stream, a);
  } else if (a.kv_fp8) {
    if (ext) hipLaunchKernelGGL((decode_mla_kernel<true, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_mla_kernel<true, false, false>), grid, block, 0, stream, a);
  } else {
    if (ext) hipLaunchKernelGGL((decode_mla_kernel<false, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_mla_kernel<false, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn
