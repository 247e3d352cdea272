// Ragged prefill over dense or paged KV, causal (bottom-right) or not, for gfx950.
//
// Computes, for every query row of every head, softmax attention over the
// keys the row may see, with the running-max / running-sum recurrence over
// key tiles ("Flywheel Attention: Attention Kernels Built for the TPU",
// section 1; "Writing Page Attention with PyPTO", section 6.3), and the
// base-2 log-sum-exp ("TokenSpeed-MLA", kernel capability summary: optional
// FP32 LSE, base-2 semantics).
//
// A workgroup owns W waves x RB blocks of 32 query rows that share one KV
// head: GH query heads of a GQA group (GH in {1, 2, 4}) times consecutive
// query tokens. Each 32-row block is 32 tokens of one head. Per key tile:
//   - the tile's K and V rows are gathered (through the block table when
//     paged, "Writing Page Attention with PyPTO", section 5.2) ahead of use
//     with direct HBM -> LDS loads (global_load_lds_dwordx4) into double
//     buffers whose 16-byte chunks are XOR-swizzled against bank conflicts;
//     keys past the request are zeroed, table entries past its last page are
//     never read (section 9);
//   - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with Q^T in registers: each lane
//     holds 16 scores of one row per 32 keys;
//   - masking (tail, and above the bottom-right causal diagonal) only on the
//     tiles that reach a row bound, decided once per tile for the wave;
//   - the row max is kept lazily: a row re-bases (and rescales O) only when
//     its max rises by more than 8 in log2 units, so P <= 2^8 ("TokenSpeed-
//     MLA", section "SM107 decode": the base is retained for rises up to 4
//     log2 units, 8 for split chunks; "Flywheel Attention", section 1: FA-4
//     skips the rescale when the max barely moves). The result is the same
//     softmax, the final division uses the same base;
//   - P rounded to bf16 (RNE) is the B operand of O^T += V^T P^T straight
//     from the score registers; V^T comes from LDS via ds_read_b64_tr_b16.
// The FP32 P sums normalise O and give the LSE. Query tiles are aligned to
// the END of each request, so tile 0 of every request sees the most keys and
// is launched first.
//
// Two kernels. prefill_pp8_kernel (D = 128): eight waves in two groups
// whose matrix and softmax phases alternate, 256 query rows per workgroup
// sharing each K/V tile. prefill_pipe_kernel (D = 64, 256): four waves, each
// software-pipelined in itself (the scores of tile j+1 on the matrix cores
// beside the softmax of tile j). Both keep separate K and V double buffers;
// D = 256 runs at one wave per SIMD (its Q operand and O accumulator take
// most of a SIMD's registers), the others at two.

#include <type_traits>

#include "attn_internal.h"
#include "device_common.h"
#include "prefill_unit.h"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// Software-pipelined kernel: four waves, one 32-row block per wave, 64-key
// tiles. Inside a wave the scores of tile j+1 are computed
// on the matrix cores while the vector units turn the scores of tile j into
// P, so neither unit waits for the other to drain. K and V have their own
// double buffers, which lets K(j+1) be resident one iteration before V(j+1):
//
//   iteration j:  wait + barrier | load K(j+2), V(j+1) | finish max S(j),
//                 re-base | S(j+1) = K(j+1) Q^T with P(j) = exp2(..) beside it |
//                 O^T += V(j)^T P(j)^T with the max over S(j+1) beside it
//
// The max over S(j+1) is taken unmasked; a tile that needs a mask masks and
// takes it again. Paged block-table entries are fetched one tile ahead of
// the loads that use them, so no load waits on a table read, and the tile
// loads are issued as inline assembly so that no LDS read in between waits
// for them (only the barrier at the top of the next iteration does).

template <int D, int W = 4>
struct PpGeom {
  static constexpr int kW = W;                         // waves per workgroup
  static constexpr int kWPE = D <= 128 ? 2 : 1;        // waves per SIMD the registers allow
  static constexpr int kRing = D <= 128 ? 0 : 4;       // LDS operand reads issued ahead (0: compiler order)
  static constexpr int kN = 64;                        // keys per tile
  static constexpr int kKB = D / 16;                   // QK k-steps
  static constexpr int kNB = D / 32;                   // PV 32-channel blocks
  static constexpr int kKK = kN / 16;                  // PV k-steps
  static constexpr int kTile = kN * D;                 // elements of one K or V tile
  static constexpr int kCPR = D / 8;                   // 16-byte chunks per row
  static constexpr int kLoads = kN * kCPR / 64 / kW;   // 1 KB direct loads per wave per tile
  static constexpr int kRowsPerInst = 64 / kCPR;       // rows one load instruction covers
  // distinct per-lane offsets: instruction k starts at row (k kW + wave) kRowsPerInst
  // and the swizzle repeats every 16 rows
  static constexpr int kLaneOffs = (kW * kRowsPerInst >= 16) ? 1 : 16 / (kW * kRowsPerInst);
  // Distinct LDS operand offsets per lane: the row swizzle permutes 16-byte
  // chunks within aligned groups of 16 (256 bytes), so K k-steps kb and
  // kb + 8 (and V channel blocks nb and nb + 4) differ by exactly 256 bytes.
  static constexpr int kKOffs = kKB > 8 ? 8 : kKB;
  static constexpr int kVOffs = kNB > 4 ? 4 : kNB;
};

// LDS byte offsets of K k-step kb and of V channel block nb for this lane.
template <int D>
__device__ __forceinline__ int pp_koff(const int (&koff)[PpGeom<D>::kKOffs], int kb) {
  return koff[kb % PpGeom<D>::kKOffs] + (kb / PpGeom<D>::kKOffs) * 256;
}
template <int D>
__device__ __forceinline__ int pp_voff(const int (&voff)[PpGeom<D>::kVOffs], int nb) {
  return voff[nb % PpGeom<D>::kVOffs] + (nb / PpGeom<D>::kVOffs) * 256;
}

// How K/V rows are addressed: dense, paged with pages of at least one tile
// (a tile then lies inside one page), or paged with smaller pages.
enum PpKv { kKvDense = 0, kKvWidePages = 1, kKvNarrowPages = 2 };

// Tile row that load k of this lane fills.
template <int D, int W = 4>
__device__ __forceinline__ int pp_row(int k, int wave, int lane) {
  using G = PpGeom<D, W>;
  return ((k * G::kW + wave) * 64 + lane) / G::kCPR;
}

// This lane's byte offsets inside the rows one load instruction covers.
// Load instruction k uses entry k % kLaneOffs: the swizzle depends on the
// row modulo 16, and instructions k and k + kLaneOffs start a multiple of
// 16 rows apart.
template <int D, int W = 4>
__device__ __forceinline__ void pp_lane_off(int wave, int lane, int64_t stride_tok,
                                            uint32_t (&off)[PpGeom<D, W>::kLaneOffs]) {
  using G = PpGeom<D, W>;
  const int r = lane / G::kCPR;
#pragma unroll
  for (int v = 0; v < G::kLaneOffs; ++v) {
    const int gchunk = (lane % G::kCPR) ^ pf_swz<D>((v * G::kW + wave) * G::kRowsPerInst + r);
    off[v] = static_cast<uint32_t>((r * stride_tok + gchunk * 8) * 2);
  }
}

// Loads of a tile that lies wholly inside the request (and, paged, inside
// one page): `tile` is its first row, wave-uniform. Load instructions KLO ..
// KHI - 1 of the wave (all by default; a range of them fills a band of rows).
template <int D, int W = 4, int KLO = 0, int KHI = PpGeom<D, W>::kLoads>
__device__ __forceinline__ void pp_issue_whole(const __bf16 *tile, int64_t stride_tok,
                                               const uint32_t (&lane_off)[PpGeom<D, W>::kLaneOffs], int wave,
                                               uint32_t lds_dst) {
  using G = PpGeom<D, W>;
#pragma unroll
  for (int k = KLO; k < KHI; ++k) {
    const int inst = k * G::kW + wave;
    lds_dma16(tile + (int64_t)inst * G::kRowsPerInst * stride_tok, lane_off[k % G::kLaneOffs], lds_dst + inst * 1024);
  }
}

// Loads of a tile row by row: rows at or past the request's end are
// zero-filled with LDS stores instead, and each row finds its page itself
// (`page` for wide pages, `pid[k]` for narrow ones).
template <int D, int KV, int W = 4, int KLO = 0, int KHI = PpGeom<D, W>::kLoads>
__device__ __forceinline__ void pp_issue_rows(const __bf16 *src, int64_t stride_page, int64_t stride_tok, int page,
                                              const int (&pid)[PpGeom<D, W>::kLoads], int j0, int lk, int pmask,
                                              int wave, int lane, __bf16 *dst) {
  using G = PpGeom<D, W>;
#pragma unroll
  for (int k = KLO; k < KHI; ++k) {
    const int inst = k * G::kW + wave;
    const int chunk_lin = inst * 64 + lane;
    const int row = chunk_lin / G::kCPR;
    const int gchunk = (chunk_lin % G::kCPR) ^ pf_swz<D>(row);
    const int j = j0 + row;
    if (j < lk) {
      const int64_t pg = (KV == kKvWidePages) ? page : (KV == kKvNarrowPages ? pid[k] : 0);
      const __bf16 *p = (KV == kKvDense) ? src + (int64_t)j * stride_tok
                                         : src + pg * stride_page + (int64_t)(j & pmask) * stride_tok;
      lds_dma16(p + gchunk * 8, lds_address(dst + inst * 512));
    } else {
      *reinterpret_cast<u32x4 *>(dst + chunk_lin * 8) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// One K or V tile: `src` is the request's first key (dense) or page 0
// (paged) of the workgroup's KV head.
template <int D, int KV, int W = 4, int KLO = 0, int KHI = PpGeom<D, W>::kLoads>
__device__ __forceinline__ void pp_issue(const __bf16 *src, int64_t stride_page, int64_t stride_tok,
                                         const uint32_t (&lane_off)[PpGeom<D, W>::kLaneOffs], int page,
                                         const int (&pid)[PpGeom<D, W>::kLoads], int j0, int lk, int pmask,
                                         int wave, int lane, __bf16 *dst) {
  if (KV != kKvNarrowPages && j0 + PpGeom<D, W>::kN <= lk) {
    const __bf16 *tile = (KV == kKvDense) ? src + (int64_t)j0 * stride_tok
                                          : src + (int64_t)page * stride_page + (int64_t)(j0 & pmask) * stride_tok;
    pp_issue_whole<D, W, KLO, KHI>(tile, stride_tok, lane_off, wave, lds_address(dst));
  } else {
    pp_issue_rows<D, KV, W, KLO, KHI>(src, stride_page, stride_tok, page, pid, j0, lk, pmask, wave, lane, dst);
  }
}

// Block-table entries for the tile at key j0 (never past the request's last
// page): one wave-uniform entry for wide pages, one per loaded row otherwise.
template <int D, int KV, int W = 4>
__device__ __forceinline__ void pp_fetch_pages(const int32_t *bt_row, int j0, int lk, int shift, int wave, int lane,
                                               int &page, int (&pid)[PpGeom<D, W>::kLoads]) {
  if constexpr (KV == kKvWidePages) {
    // a scalar load (the table is read-only here): waiting for it does not
    // wait for the vector-memory tile loads in flight
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    page = (j0 < lk) ? reinterpret_cast<const_i32 *>(reinterpret_cast<uintptr_t>(bt_row))[j0 >> shift] : 0;
  } else if constexpr (KV == kKvNarrowPages) {
#pragma unroll
    for (int k = 0; k < PpGeom<D, W>::kLoads; ++k) {
      const int j = j0 + pp_row<D, W>(k, wave, lane);
      pid[k] = (j < lk) ? bt_row[j >> shift] : 0;
    }
  }
}

// S^T for the 64 keys of a resident K tile: two 32-key blocks, 16 scores of
// this lane's row each.
template <int D>
__device__ __forceinline__ void pp_scores(const char *kbytes, const int (&koff)[PpGeom<D>::kKOffs],
                                          const bf16x8 (&qop)[PpGeom<D>::kKB], f32x16 (&s)[2]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    s[sub] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < PpGeom<D>::kKB; ++kb)
      s[sub] = mfma32x32x16(*reinterpret_cast<const bf16x8 *>(kbytes + pp_koff<D>(koff, kb) + sub * 32 * D * 2),
                            qop[kb], s[sub]);
  }
}

__device__ __forceinline__ float pp_max(const f32x16 (&s)[2]) {
  float mx = kNegInf;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sub][i]);
  return mx;
}

// Keys at or past `bound`, or before `begin` (this lane's row), get -inf.
__device__ __forceinline__ void pp_mask(f32x16 (&s)[2], int j0, int begin, int bound, int h) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + 32 * sub + 8 * (i >> 2) + 4 * h + (i & 3);
      s[sub][i] = (j < bound && j >= begin) ? s[sub][i] : kNegInf;
    }
}

// One tile's P, sum and O update, and the scores (with their unmasked max)
// of the following tile from the K tile in `knext`.
template <int D>
__device__ __forceinline__ void pp_step(f32x16 (&s)[2], float &mx, float m_use, float c, float alpha, float &lsum,
                                        f32x16 (&oacc)[PpGeom<D>::kNB], const char *knext, const char *vbytes,
                                        const int (&koff)[PpGeom<D>::kKOffs], const int (&voff)[2][PpGeom<D>::kVOffs],
                                        const bf16x8 (&qop)[PpGeom<D>::kKB]) {
  using G = PpGeom<D>;
  if constexpr (G::kRing == 0) {
    f32x16 sn[2];
    pp_scores<D>(knext, koff, qop, sn);
    bf16x8 pop[G::kKK];
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pe = exp2_fast(__builtin_fmaf(s[sub][i], c, -m_use));
        pop[2 * sub + (i >> 3)][i & 7] = to_bf16(pe);
        ps[i & 1] += pe;
      }
#pragma unroll
    for (int kk = 0; kk < G::kKK; ++kk)
#pragma unroll
      for (int nb = 0; nb < G::kNB; ++nb) {
        const bf16x4 lo = lds_read_tr16(vbytes + pp_voff<D>(voff[0], nb) + kk * 16 * D * 2);
        const bf16x4 hi = lds_read_tr16(vbytes + pp_voff<D>(voff[1], nb) + kk * 16 * D * 2);
        oacc[nb] = mfma32x32x16(concat(lo, hi), pop[kk], oacc[nb]);
      }
    lsum = alpha * lsum + (ps[0] + ps[1]);
    s[0] = sn[0];
    s[1] = sn[1];
    mx = pp_max(s);
  } else {
    // LDS operand reads run kRing MFMAs ahead in a register ring; the exp
    // work of the current tile is spread over the QK steps and the max of
    // the next tile's scores over the PV steps (one wave per SIMD at this D
    // leaves no other wave to hide LDS latency behind).
    constexpr int kQK = 2 * G::kKB;
    constexpr int kPV = G::kKK * G::kNB;
    constexpr int kSteps = kQK + kPV;
    constexpr int kR = G::kRing;
    constexpr int kExpPer = 32 / kQK;
    constexpr int kMaxPer = 32 / kPV;
    auto rd = [&](int t) -> bf16x8 {
      if (t < kQK)
        return *reinterpret_cast<const bf16x8 *>(knext + pp_koff<D>(koff, t % G::kKB) + (t / G::kKB) * 32 * D * 2);
      const int u = t - kQK, kk = u / G::kNB, nb = u % G::kNB;
      return concat(lds_read_tr16(vbytes + pp_voff<D>(voff[0], nb) + kk * 16 * D * 2),
                    lds_read_tr16(vbytes + pp_voff<D>(voff[1], nb) + kk * 16 * D * 2));
    };
    bf16x8 ring[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) ring[i] = rd(i);
    f32x16 sn[2] = {f32x16{}, f32x16{}};
    bf16x8 pop[G::kKK];
    float ps[2] = {0.f, 0.f};
    float mxn = kNegInf;
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      if (t < kQK) {
        sn[t / G::kKB] = mfma32x32x16(ring[t % kR], qop[t % G::kKB], sn[t / G::kKB]);
#pragma unroll
        for (int e = 0; e < kExpPer; ++e) {
          const int idx = t * kExpPer + e, sb = idx / 16, i = idx % 16;
          const float pe = exp2_fast(__builtin_fmaf(s[sb][i], c, -m_use));
          pop[2 * sb + (i >> 3)][i & 7] = to_bf16(pe);
          ps[i & 1] += pe;
        }
      } else {
        const int u = t - kQK;
        oacc[u % G::kNB] = mfma32x32x16(ring[t % kR], pop[u / G::kNB], oacc[u % G::kNB]);
#pragma unroll
        for (int e = 0; e < kMaxPer; ++e) {
          const int idx = u * kMaxPer + e;
          mxn = fmaxf(mxn, sn[idx / 16][idx % 16]);
        }
      }
      if (t + kR < kSteps) ring[t % kR] = rd(t + kR);
    }
    __builtin_amdgcn_sched_barrier(0);
    lsum = alpha * lsum + (ps[0] + ps[1]);
    s[0] = sn[0];
    s[1] = sn[1];
    mx = mxn;
  }
}

template <int D, int KV>
__global__ __launch_bounds__(64 * PpGeom<D>::kW, PpGeom<D>::kWPE) void prefill_pipe_kernel(const PrefillArgs a) {
  using G = PpGeom<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[4 * G::kTile];   // K slot 0, K slot 1, V slot 0, V slot 1
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int r32 = lane & 31;

  PfUnit u;
  if (!pf_unit(a, G::kW, u)) return;
  const int blocks_per_head = G::kW / u.gh;
  const int head = u.h0 + wave / blocks_per_head;
  const int t = u.q_end - u.tq + (wave % blocks_per_head) * 32 + r32;   // may be < 0 at the top
  const bool row_valid = t >= u.q_begin && t < u.q_end;
  int bound = a.causal ? min(u.lk, max(0, u.lk - u.lq + t + 1)) : u.lk;
  if (!row_valid) bound = 0;
  // Sliding window ("TokenSpeed-MLA", kernel capability summary,
  // window_left): row t sees no key before lk - lq - window_left + t. The
  // workgroup's walk starts at the tile holding its first row's first key.
  const bool windowed = a.window_left >= 0;
  const int begin = windowed ? max(0, u.lk - u.lq - a.window_left + t) : 0;
  // The workgroup's keys: from the tile holding its first row's first key,
  // within its split (splits are whole tiles) when the keys are split.
  int jb = windowed ? max(0, u.lk - u.lq - a.window_left + u.q_begin) & ~(G::kN - 1) : 0;
  int split_end = 0x7fffffff;
  if (a.kv_splits > 1) {
    jb = max(jb, u.split * a.split_tokens);
    split_end = (u.split + 1) * a.split_tokens;
  }
  int wave_max = bound, valid_min = row_valid ? bound : 0x7fffffff;
  int begin_max = row_valid ? begin : 0, begin_min = row_valid ? begin : 0x7fffffff;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    wave_max = max(wave_max, __shfl_xor(wave_max, off, 64));
    valid_min = min(valid_min, __shfl_xor(valid_min, off, 64));
    begin_max = max(begin_max, __shfl_xor(begin_max, off, 64));
    begin_min = min(begin_min, __shfl_xor(begin_min, off, 64));
  }
  wave_max = __builtin_amdgcn_readfirstlane(wave_max);
  valid_min = __builtin_amdgcn_readfirstlane(valid_min);
  begin_max = __builtin_amdgcn_readfirstlane(begin_max);
  begin_min = __builtin_amdgcn_readfirstlane(begin_min);
  const int kv_end = min(split_end, a.causal ? min(u.lk, max(0, u.lk - u.lq + u.q_end)) : u.lk);
  const int nt = kv_end > jb ? (kv_end - jb + G::kN - 1) / G::kN : 0;       // tiles the workgroup loads
  // tiles this wave computes (<= nt)
  const int ntw = min(nt, wave_max > jb ? (wave_max - jb + G::kN - 1) / G::kN : 0);
  // the wave's first tile with a key for one of its rows (0 without a window)
  const int it0 = (windowed && begin_min != 0x7fffffff && begin_min > jb) ? (begin_min - jb) / G::kN : 0;

  // Q^T operands (a negative scale negates Q, exact in bf16, so c > 0)
  const float c = fabsf(a.scale_log2);
  const u32x4 qsign = (a.scale_log2 < 0.f) ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u} : u32x4{};
  bf16x8 qop[G::kKB];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + (u.q_off + t) * a.q_stride_tok +
                         (int64_t)head * a.q_stride_head;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
      qop[kb] = row_valid ? __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, load_bf16x8(qrow + kb * 16 + h * 8)) ^ qsign)
                          : bf16x8{};
  }
  int koff[G::kKOffs];
  {
    const int hf = h ^ pf_swz<D>(r32);
#pragma unroll
    for (int kb = 0; kb < G::kKOffs; ++kb) koff[kb] = r32 * D * 2 + ((2 * kb) ^ hf) * 16;
  }
  int voff[2][G::kVOffs];
  {
    const int s16 = lane & 15;
    const int row0 = 4 * h + (s16 >> 2);
    const int cb = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
    const int f0 = pf_swz<D>(row0), f1 = pf_swz<D>(row0 + 8);
#pragma unroll
    for (int nb = 0; nb < G::kVOffs; ++nb) {
      voff[0][nb] = row0 * D * 2 + ((4 * nb + cb) ^ f0) * 16 + 8 * (s16 & 1);
      voff[1][nb] = (row0 + 8) * D * 2 + ((4 * nb + cb) ^ f1) * 16 + 8 * (s16 & 1);
    }
  }

  // KV sources of the workgroup's head
  const __bf16 *ksrc = static_cast<const __bf16 *>(a.k) + (int64_t)u.kvh * a.k_stride_head;
  const __bf16 *vsrc = static_cast<const __bf16 *>(a.v) + (int64_t)u.kvh * a.v_stride_head;
  if constexpr (KV == kKvDense) {
    ksrc += u.kv_off * a.k_stride_tok;
    vsrc += u.kv_off * a.v_stride_tok;
  }
  uint32_t koff_g[G::kLaneOffs], voff_g[G::kLaneOffs];
  pp_lane_off<D>(wave, lane, a.k_stride_tok, koff_g);
  pp_lane_off<D>(wave, lane, a.v_stride_tok, voff_g);
  const int32_t *bt_row = (KV != kKvDense) ? a.block_table + (int64_t)u.b * a.block_table_stride : nullptr;
  const int pmask = (1 << a.page_shift) - 1;
  // Table entries of the next K tile (it+2) and V tile (it+1) to load, each
  // fetched into its own registers one iteration before use.
  int kpage = 0, vpage = 0;
  int kpid[G::kLoads] = {}, vpid[G::kLoads] = {};
  auto issue_k = [&](int j0t, int page, const int (&pid)[G::kLoads], __bf16 *dst) {
    pp_issue<D, KV>(ksrc, a.k_stride_page, a.k_stride_tok, koff_g, page, pid, j0t, u.lk, pmask, wave, lane, dst);
  };
  auto issue_v = [&](int j0t, int page, const int (&pid)[G::kLoads], __bf16 *dst) {
    pp_issue<D, KV>(vsrc, a.v_stride_page, a.v_stride_tok, voff_g, page, pid, j0t, u.lk, pmask, wave, lane, dst);
  };

  auto kslot = [&](int par) { return lds + par * G::kTile; };
  auto vslot = [&](int par) { return lds + (2 + par) * G::kTile; };
  if (nt > 0) {
    pp_fetch_pages<D, KV>(bt_row, jb, u.lk, a.page_shift, wave, lane, kpage, kpid);
    issue_k(jb, kpage, kpid, kslot(0));
    issue_v(jb, kpage, kpid, vslot(0));
    pp_fetch_pages<D, KV>(bt_row, jb + G::kN, u.lk, a.page_shift, wave, lane, vpage, vpid);
    if (nt > 1) issue_k(jb + G::kN, vpage, vpid, kslot(1));
    pp_fetch_pages<D, KV>(bt_row, jb + 2 * G::kN, u.lk, a.page_shift, wave, lane, kpage, kpid);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  f32x16 s[2];
  float mx = kNegInf;
  if (ntw > 0) {
    pp_scores<D>(reinterpret_cast<const char *>(kslot(0)), koff, qop, s);
    mx = pp_max(s);
  }
  float m = kNegInf, lsum = 0.f;
  f32x16 oacc[G::kNB];
#pragma unroll
  for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] = f32x16{};

  // The loop is unrolled by two so each half knows its LDS slots at compile
  // time; the per-lane offsets are made opaque once per tile, so the compiler
  // folds every slot and block constant into the LDS reads' immediate offsets
  // rather than computing addresses per tile or keeping each one in a register.
  auto tile_step = [&](int it, auto par_c) {
    constexpr int par = decltype(par_c)::value;
#pragma unroll
    for (int kb = 0; kb < G::kKOffs; ++kb) asm volatile("" : "+v"(koff[kb]));
#pragma unroll
    for (int nb = 0; nb < G::kVOffs; ++nb) asm volatile("" : "+v"(voff[0][nb]), "+v"(voff[1][nb]));
    // K(it+1) and V(it) have landed for every wave, and every wave is done
    // with K(it) and V(it-1), whose slots take K(it+2) and V(it+1).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int j0 = jb + it * G::kN;
    if (it + 2 < nt) issue_k(j0 + 2 * G::kN, kpage, kpid, kslot(par));
    if (it + 1 < nt) issue_v(j0 + G::kN, vpage, vpid, vslot(par ^ 1));
    if constexpr (KV != kKvDense) {
      if (it + 2 < nt) pp_fetch_pages<D, KV>(bt_row, j0 + 2 * G::kN, u.lk, a.page_shift, wave, lane, vpage, vpid);
      if (it + 3 < nt) pp_fetch_pages<D, KV>(bt_row, j0 + 3 * G::kN, u.lk, a.page_shift, wave, lane, kpage, kpid);
    }
    // A wave whose rows' window starts in tile it0 skips the tiles before
    // it0 - 1; on tile it0 - 1 every key is below every row's window, so the
    // mask clears the stale scores, the step adds nothing and computes the
    // scores of tile it0. (0 <= it0 < ntw when ntw > 0: a valid row's first
    // key lies below its bound; one unsigned compare tests it0 - 1 <= it < ntw.)
    // Stepping every wave through every tile instead (masked whole) ran 3-4 %
    // slower at D = 256.
    if ((unsigned)(it + 1 - it0) < (unsigned)(ntw + 1 - it0)) {
      if (j0 + G::kN > valid_min || j0 < begin_max) {
        pp_mask(s, j0, begin, bound, h);
        mx = pp_max(s);
      }
      const float mt = half_max(mx) * c;
      const float m_new = (mt > m + kRebase) ? mt : m;    // keep the base unless the max rose by > kRebase
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);          // 1 when kept; 0 from -inf
      m = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] *= alpha;
      }
      const char *knext = reinterpret_cast<const char *>(kslot(par ^ 1));
      const char *vbytes = reinterpret_cast<const char *>(vslot(par));
      // The scores of tile it+1 are computed even on the wave's last tile
      // (from whatever that LDS slot holds) and then dropped: one branch-free
      // body keeps the exp work beside the MFMAs.
      pp_step<D>(s, mx, m_use, c, alpha, lsum, oacc, knext, vbytes, koff, voff, qop);
    }
  };
  for (int it = 0; it < nt; it += 2) {
    tile_step(it, std::integral_constant<int, 0>{});
    if (it + 1 < nt) tile_step(it + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O / l -> bf16; LSE2 = m + log2(l) ----
  const float l = half_sum(lsum);
  if (!row_valid) return;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  if (a.kv_splits > 1) {
    // this split's normalised partial (FP32) and LSE, merged by the LSE
    // reducer; a split without keys for the row leaves only its -inf LSE
    const int64_t rows = (int64_t)a.total_q * a.num_q_heads;
    const int64_t r = (u.q_off + t) * a.num_q_heads + head;
    if (u.q_off + t >= a.total_q) return;              // total_q too small: outside the workspace
    if (h == 0) a.lse_parts[u.split * rows + r] = (l > 0.f) ? ((m == kNegInf) ? 0.f : m) + __log2f(l) : kNegInf;
    if (l > 0.f) {
      float *prow = a.o_parts + (u.split * rows + r) * D;
#pragma unroll
      for (int nb = 0; nb < G::kNB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = oacc[nb][4 * g + i] * inv;
          *reinterpret_cast<f32x4 *>(prow + 32 * nb + 8 * g + 4 * h) = ov;
        }
    }
    return;
  }
  __bf16 *orow = static_cast<__bf16 *>(a.o) + (u.q_off + t) * a.o_stride_tok + (int64_t)head * a.o_stride_head;
#pragma unroll
  for (int nb = 0; nb < G::kNB; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = to_bf16(oacc[nb][4 * g + i] * inv);
      *reinterpret_cast<u32x2 *>(orow + 32 * nb + 8 * g + 4 * h) = __builtin_bit_cast(u32x2, ob);
    }
  if (a.lse && h == 0) {
    const float muse = (m == kNegInf) ? 0.f : m;
    a.lse[(u.q_off + t) * a.num_q_heads + head] = (l > 0.f) ? muse + __log2f(l) : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong kernel (D = 128): eight waves of one 32-row block each, in two
// groups of four; waves w and w + 4 run on the same SIMD. A tile step splits
// into a matrix phase (S(j+1) = K(j+1) Q^T and O^T += V(j)^T P(j)^T: 32
// MFMAs, operands from LDS) and a vector phase (mask, max and re-base of
// S(j+1), P(j+1) = exp2(..), sums), and the two groups run them out of step,
// separated by workgroup barriers: while one group's waves keep the matrix
// cores busy, the other group's waves on the same SIMDs do their softmax
// ("Flywheel Attention", section 3.1: the exp work of one fragment beside
// the matrix work of another). Per tile j:
//
//   barrier (tile loads landed) | group 0: matrix j   group 1: vector j-1 |
//   barrier                     | group 0: vector j   group 1: matrix j
//
// The waves of the matrix phase raise their issue priority. 256 query rows
// share each K/V tile, and a CU holds one workgroup (two waves per SIMD).

template <int D>
struct P8Geom {
  static constexpr int kW = 8;                // waves per workgroup (two groups of four)
  static constexpr int kN = 64;               // keys per tile
  static constexpr int kKB = D / 16;          // QK k-steps
  static constexpr int kNB = D / 32;          // PV 32-channel blocks
  static constexpr int kKK = kN / 16;         // PV k-steps
  static constexpr int kTile = kN * D;        // elements of one K or V tile
  static constexpr int kRing = 3;             // LDS operand reads in flight ahead of the MFMAs
};

template <int D, int KV>
__global__ __launch_bounds__(64 * P8Geom<D>::kW, 1) void prefill_pp8_kernel(const PrefillArgs a) {
  using G = P8Geom<D>;
  using L = PpGeom<D, 4>;                     // the tile loads, spread over the four waves of group 0
  static_assert(L::kN == G::kN, "tile size");
  __shared__ __attribute__((aligned(16))) __bf16 lds[4 * G::kTile];   // K slot 0, K slot 1, V slot 0, V slot 1
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;                  // 0: matrix phase first; 1: vector phase first
  const int h = lane >> 5;
  const int r32 = lane & 31;

  PfUnit u;
  if (!pf_unit(a, G::kW, u)) return;
  const int blocks_per_head = G::kW / u.gh;
  const int head = u.h0 + wave / blocks_per_head;
  const int t = u.q_end - u.tq + (wave % blocks_per_head) * 32 + r32;   // may be < 0 at the top
  const bool row_valid = t >= u.q_begin && t < u.q_end;
  int bound = a.causal ? min(u.lk, max(0, u.lk - u.lq + t + 1)) : u.lk;
  if (!row_valid) bound = 0;
  // Sliding window ("TokenSpeed-MLA", kernel capability summary,
  // window_left): row t sees no key before lk - lq - window_left + t.
  const bool windowed = a.window_left >= 0;
  const int begin = windowed ? max(0, u.lk - u.lq - a.window_left + t) : 0;
  int jb = windowed ? max(0, u.lk - u.lq - a.window_left + u.q_begin) & ~(G::kN - 1) : 0;
  int split_end = 0x7fffffff;
  if (a.kv_splits > 1) {
    jb = max(jb, u.split * a.split_tokens);
    split_end = (u.split + 1) * a.split_tokens;
  }
  int wave_max = bound, valid_min = row_valid ? bound : 0x7fffffff;
  int begin_max = row_valid ? begin : 0, begin_min = row_valid ? begin : 0x7fffffff;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    wave_max = max(wave_max, __shfl_xor(wave_max, off, 64));
    valid_min = min(valid_min, __shfl_xor(valid_min, off, 64));
    begin_max = max(begin_max, __shfl_xor(begin_max, off, 64));
    begin_min = min(begin_min, __shfl_xor(begin_min, off, 64));
  }
  wave_max = __builtin_amdgcn_readfirstlane(wave_max);
  valid_min = __builtin_amdgcn_readfirstlane(valid_min);
  begin_max = __builtin_amdgcn_readfirstlane(begin_max);
  begin_min = __builtin_amdgcn_readfirstlane(begin_min);
  const int kv_end = min(split_end, a.causal ? min(u.lk, max(0, u.lk - u.lq + u.q_end)) : u.lk);
  const int nt = kv_end > jb ? (kv_end - jb + G::kN - 1) / G::kN : 0;       // tiles the workgroup loads
  const int ntw = min(nt, wave_max > jb ? (wave_max - jb + G::kN - 1) / G::kN : 0);   // tiles this wave computes
  // the wave's first tile with a key for one of its rows (0 without a
  // window); its matrix phases start one tile earlier (that tile's keys are
  // all below every row's window: the vector phase before it masks the
  // stale scores whole, so it adds nothing, and it computes the scores of
  // tile it0)
  const int it0 = (windowed && begin_min != 0x7fffffff && begin_min > jb) ? (begin_min - jb) / G::kN : 0;
  // (at most tile 1: the prologue holds K(0) and K(1); the tiles between
  // it_lo and it0 - 1 are masked whole and add nothing)
  const int it_lo = min(max(it0 - 1, 0), 1);

  // Q^T operands (a negative scale negates Q, exact in bf16, so c > 0)
  const float c = fabsf(a.scale_log2);
  const u32x4 qsign = (a.scale_log2 < 0.f) ? u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u} : u32x4{};
  bf16x8 qop[G::kKB];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + (u.q_off + t) * a.q_stride_tok +
                         (int64_t)head * a.q_stride_head;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
      qop[kb] = row_valid ? __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, load_bf16x8(qrow + kb * 16 + h * 8)) ^ qsign)
                          : bf16x8{};
  }
  int koff[G::kKB];
  {
    const int hf = h ^ pf_swz<D>(r32);
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb) koff[kb] = r32 * D * 2 + ((2 * kb) ^ hf) * 16;
  }
  int voff[2][G::kNB];
  {
    const int s16 = lane & 15;
    const int row0 = 4 * h + (s16 >> 2);
    const int cb = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
    const int f0 = pf_swz<D>(row0), f1 = pf_swz<D>(row0 + 8);
#pragma unroll
    for (int nb = 0; nb < G::kNB; ++nb) {
      voff[0][nb] = row0 * D * 2 + ((4 * nb + cb) ^ f0) * 16 + 8 * (s16 & 1);
      voff[1][nb] = (row0 + 8) * D * 2 + ((4 * nb + cb) ^ f1) * 16 + 8 * (s16 & 1);
    }
  }

  const __bf16 *ksrc = static_cast<const __bf16 *>(a.k) + (int64_t)u.kvh * a.k_stride_head;
  const __bf16 *vsrc = static_cast<const __bf16 *>(a.v) + (int64_t)u.kvh * a.v_stride_head;
  if constexpr (KV == kKvDense) {
    ksrc += u.kv_off * a.k_stride_tok;
    vsrc += u.kv_off * a.v_stride_tok;
  }
  const int lw = wave & 3;                    // the wave's share of the tile loads (group 0 loads)
  uint32_t koff_g[L::kLaneOffs], voff_g[L::kLaneOffs];
  pp_lane_off<D, 4>(lw, lane, a.k_stride_tok, koff_g);
  pp_lane_off<D, 4>(lw, lane, a.v_stride_tok, voff_g);
  const int32_t *bt_row = (KV != kKvDense) ? a.block_table + (int64_t)u.b * a.block_table_stride : nullptr;
  const int pmask = (1 << a.page_shift) - 1;
  int kpage = 0, vpage = 0;
  int kpid[L::kLoads] = {}, vpid[L::kLoads] = {};
  auto issue_k = [&](int j0t, int page, const int (&pid)[L::kLoads], __bf16 *dst) __attribute__((always_inline)) {
    pp_issue<D, KV, 4>(ksrc, a.k_stride_page, a.k_stride_tok, koff_g, page, pid, j0t, u.lk, pmask, lw, lane, dst);
  };
  auto issue_v = [&](int j0t, int page, const int (&pid)[L::kLoads], __bf16 *dst) __attribute__((always_inline)) {
    pp_issue<D, KV, 4>(vsrc, a.v_stride_page, a.v_stride_tok, voff_g, page, pid, j0t, u.lk, pmask, lw, lane, dst);
  };
  auto kslot = [&](int par) { return lds + par * G::kTile; };
  auto vslot = [&](int par) { return lds + (2 + par) * G::kTile; };
  if (grp == 0 && nt > 0) {
    pp_fetch_pages<D, KV, 4>(bt_row, jb, u.lk, a.page_shift, lw, lane, kpage, kpid);
    issue_k(jb, kpage, kpid, kslot(0));
    issue_v(jb, kpage, kpid, vslot(0));
    pp_fetch_pages<D, KV, 4>(bt_row, jb + G::kN, u.lk, a.page_shift, lw, lane, vpage, vpid);
    if (nt > 1) issue_k(jb + G::kN, vpage, vpid, kslot(1));
    pp_fetch_pages<D, KV, 4>(bt_row, jb + 2 * G::kN, u.lk, a.page_shift, lw, lane, kpage, kpid);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  f32x16 sn[2] = {f32x16{}, f32x16{}};        // scores of the next tile
  bf16x8 pop[G::kKK];                         // P of the current tile, bf16
  float m = kNegInf, lsum = 0.f;
  f32x16 oacc[G::kNB];
#pragma unroll
  for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < G::kKK; ++kk) pop[kk] = bf16x8{};

  // Matrix phase j: S(j+1) = K(j+1) Q^T from `knext`, O^T += V(j)^T P(j)^T
  // from `vbytes`; one LDS operand read per MFMA, issued kRing ahead.
  auto matrix_phase = [&](const char *knext, const char *vbytes) __attribute__((always_inline)) {
    constexpr int kQK = 2 * G::kKB, kPV = G::kKK * G::kNB, kSteps = kQK + kPV, kR = G::kRing;
    auto rd = [&](int q) __attribute__((always_inline)) -> bf16x8 {
      if (q < kQK) return *reinterpret_cast<const bf16x8 *>(knext + koff[q % G::kKB] + (q / G::kKB) * 32 * D * 2);
      const int v = q - kQK, kk = v / G::kNB, nb = v % G::kNB;
      return concat(lds_read_tr16(vbytes + voff[0][nb] + kk * 16 * D * 2),
                    lds_read_tr16(vbytes + voff[1][nb] + kk * 16 * D * 2));
    };
    __builtin_amdgcn_s_setprio(1);
    bf16x8 ring[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) ring[i] = rd(i);
    sn[0] = f32x16{};
    sn[1] = f32x16{};
#pragma unroll
    for (int q = 0; q < kSteps; ++q) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 op = ring[q % kR];
      if (q + kR < kSteps) ring[q % kR] = rd(q + kR);
      if (q < kQK) {
        sn[q / G::kKB] = mfma32x32x16(op, qop[q % G::kKB], sn[q / G::kKB]);
      } else {
        const int v = q - kQK;
        oacc[v % G::kNB] = mfma32x32x16(op, pop[v / G::kNB], oacc[v % G::kNB]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Vector phase for the scores of the tile at key j0n: mask (on tiles that
  // reach a row bound), lazy re-base of the row max (O rescaled only when it
  // rises by more than kRebase), P = exp2(s c - m) rounded to bf16, sums.
  auto vector_phase = [&](int j0n) __attribute__((always_inline)) {
    if (j0n + G::kN > valid_min || j0n < begin_max) pp_mask(sn, j0n, begin, bound, h);
    const float mt = half_max(pp_max(sn)) * c;
    const float m_new = (mt > m + kRebase) ? mt : m;   // keep the base unless the max rose by > kRebase
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);          // 1 when kept; 0 from -inf
    m = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] *= alpha;
    }
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pe = exp2_fast(__builtin_fmaf(sn[sub][i], c, -m_use));
        pop[2 * sub + (i >> 3)][i & 7] = to_bf16(pe);
        ps[i & 1] += pe;
      }
    lsum = alpha * lsum + (ps[0] + ps[1]);
  };

  // The scores of the wave's first tile (K(0) or K(1), both resident).
  if (it_lo < ntw) {
    const char *k0 = reinterpret_cast<const char *>(kslot(it_lo & 1));
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
        sn[sub] = mfma32x32x16(*reinterpret_cast<const bf16x8 *>(k0 + koff[kb] + sub * 32 * D * 2), qop[kb], sn[sub]);
  }
  // Both groups run the same sequence, group 1 one phase behind:
  //   group 0:  V(0) | B M(0) B V(1) | B M(1) B V(2) | ... | B
  //   group 1:  B V(0) | B M(0) B V(1) | B M(1) B V(2) | ...
  // (B a workgroup barrier, M(j) the matrix phase of tile j, V(j) the vector
  // phase of the scores of tile j). Between two barriers one group is in a
  // matrix phase and the other in a vector phase. Only group 0 loads tiles:
  // at the barrier before its M(j), K(j) and V(j-1) have been read by both
  // groups' M(j-1), and the loads it issues there (K(j+2), V(j+1)) land
  // before the barrier before its M(j+1), which group 1's M(j+1) follows.
  auto vec = [&](int j) __attribute__((always_inline)) {
    if (j >= it_lo && j < ntw) vector_phase(jb + j * G::kN);
  };
  if (grp == 0) vec(0);
  else {
    __syncthreads();
    vec(0);
  }
  for (int it = 0; it < nt; ++it) {
    if (grp == 0) {
      // this wave's loads of K(it+1) and V(it) (issued a tile ago) have landed
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (grp == 0) {
      const int j0 = jb + it * G::kN;
      if (it + 2 < nt) issue_k(j0 + 2 * G::kN, kpage, kpid, kslot(it & 1));
      if (it + 1 < nt) issue_v(j0 + G::kN, vpage, vpid, vslot((it + 1) & 1));
      if constexpr (KV != kKvDense) {
        if (it + 2 < nt)
          pp_fetch_pages<D, KV, 4>(bt_row, j0 + 2 * G::kN, u.lk, a.page_shift, lw, lane, vpage, vpid);
        if (it + 3 < nt)
          pp_fetch_pages<D, KV, 4>(bt_row, j0 + 3 * G::kN, u.lk, a.page_shift, lw, lane, kpage, kpid);
      }
    }
    if (it >= it_lo && it < ntw)
      matrix_phase(reinterpret_cast<const char *>(kslot((it + 1) & 1)), reinterpret_cast<const char *>(vslot(it & 1)));
    __syncthreads();
    vec(it + 1);
  }
  if (grp == 0) __syncthreads();

  // ---- epilogue: O / l -> bf16; LSE2 = m + log2(l) ----
  const float l = half_sum(lsum);
  if (!row_valid) return;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  if (a.kv_splits > 1) {
    const int64_t rows = (int64_t)a.total_q * a.num_q_heads;
    const int64_t r = (u.q_off + t) * a.num_q_heads + head;
    if (u.q_off + t >= a.total_q) return;              // total_q too small: outside the workspace
    if (h == 0) a.lse_parts[u.split * rows + r] = (l > 0.f) ? ((m == kNegInf) ? 0.f : m) + __log2f(l) : kNegInf;
    if (l > 0.f) {
      float *prow = a.o_parts + (u.split * rows + r) * D;
#pragma unroll
      for (int nb = 0; nb < G::kNB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = oacc[nb][4 * g + i] * inv;
          *reinterpret_cast<f32x4 *>(prow + 32 * nb + 8 * g + 4 * h) = ov;
        }
    }
    return;
  }
  __bf16 *orow = static_cast<__bf16 *>(a.o) + (u.q_off + t) * a.o_stride_tok + (int64_t)head * a.o_stride_head;
#pragma unroll
  for (int nb = 0; nb < G::kNB; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = to_bf16(oacc[nb][4 * g + i] * inv);
      *reinterpret_cast<u32x2 *>(orow + 32 * nb + 8 * g + 4 * h) = __builtin_bit_cast(u32x2, ob);
    }
  if (a.lse && h == 0) {
    const float muse = (m == kNegInf) ? 0.f : m;
    a.lse[(u.q_off + t) * a.num_q_heads + head] = (l > 0.f) ? muse + __log2f(l) : kNegInf;
  }
}

template <int D, int KV>
hipError_t launch_pp(const PrefillArgs &a, hipStream_t stream) {
  using G = PpGeom<D>;
  constexpr bool kPing = D == 128;
  constexpr int kWaves = kPing ? P8Geom<D>::kW : G::kW;
  const int gh = pf_heads_per_wg(a.num_q_heads / a.num_kv_heads);
  const int tq = 32 * kWaves / gh;
  const int64_t q_tiles = (a.max_seqlen_q + tq - 1) / tq;
  const int64_t blocks = q_tiles * (a.kv_splits > 1 ? a.kv_splits : 1) * a.batch * (a.num_q_heads / gh);
  if constexpr (kPing)
    hipLaunchKernelGGL((prefill_pp8_kernel<D, KV>), dim3((unsigned)blocks), dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_pipe_kernel<D, KV>), dim3((unsigned)blocks), dim3(64 * G::kW), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.kv_splits <= 1) return err;
  MergeArgs m{};
  m.o_parts = a.o_parts;
  m.lse_parts = a.lse_parts;
  m.num_splits = a.kv_splits;
  m.num_rows = (int64_t)a.total_q * a.num_q_heads;
  m.head_dim_v = D;
  m.o = a.o;
  m.o_bf16 = 1;
  m.lse = a.lse;
  return launch_merge(m, stream);
}

template <int D>
hipError_t launch_pp_kv(const PrefillArgs &a, hipStream_t stream) {
  if (!a.block_table) return launch_pp<D, kKvDense>(a, stream);
  if ((1 << a.page_shift) >= PpGeom<D>::kN) return launch_pp<D, kKvWidePages>(a, stream);
  return launch_pp<D, kKvNarrowPages>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_pp_kv<64>(a, stream);
    case 128: return launch_pp_kv<128>(a, stream);
    case 256: return launch_pp_kv<256>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace attn
