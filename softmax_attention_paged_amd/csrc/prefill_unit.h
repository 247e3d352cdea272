// Pieces the prefill kernels share: the work unit a workgroup owns, the LDS
// swizzle of bf16 tiles, and the lazy re-base threshold. Internal header.
#pragma once

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

constexpr float kRebase = 8.0f;   // log2 units a row max may rise before the row re-bases

// LDS tiles are unpadded [keys][D] with the 16-byte chunks of row r stored at
// slot chunk ^ f(r). f spreads the 16 rows a K-operand read touches over all
// 64 banks, and gives the 4 rows x 4 chunks of a transposing V read (32
// lanes) distinct banks too.
template <int D>
__device__ __forceinline__ int pf_swz(int row) {
  if constexpr (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

struct PfUnit {
  int b, kvh, h0;              // request, KV head, first query head of the workgroup
  int gh, tq;                  // query heads and query tokens per workgroup
  int q_begin, q_end;          // query rows of the request covered by this workgroup (relative)
  int lq, lk;                  // request lengths
  int64_t q_off;               // first query token of the request in the packed Q
  int64_t kv_off;              // dense: first key of the request in packed K/V
  int split;                   // the workgroup's split of the keys (0 without splits)
};

// Heads per workgroup for a GQA group: the largest of 4, 2, 1 dividing it.
__host__ __device__ __forceinline__ int pf_heads_per_wg(int group) {
  return (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
}

// The rows workgroup blockIdx.x owns when it holds `blocks` 32-row blocks:
// gh heads of one KV group times tq = 32 blocks / gh tokens, tiles counted
// from the end of the request, and with key splits the split it walks. The
// head group is the fastest index, so with a head-group count that is a
// multiple of 8 every workgroup of one KV head lands on the same XCD (blocks
// go to the XCDs in turn) and shares its L2. Without splits the query tile
// comes next (the longest rows of every request start first). With splits
// the split is slowest (the workgroups running together walk the same key
// range of as many query tiles as without splits) and the request is slower
// than the query tile: workgroups that stream the same keys are launched
// back to back, and slots that free together take the tiles of one request
// and split, so the workgroups sharing a K/V tile in L2 start together round
// after round rather than drifting apart. False when the request has no
// tile of that index.
__device__ __forceinline__ bool pf_unit(const PrefillArgs &a, int blocks, PfUnit &u) {
  const int group = a.num_q_heads / a.num_kv_heads;
  u.gh = pf_heads_per_wg(group);
  u.tq = 32 * (blocks / u.gh);
  const int head_groups = a.num_q_heads / u.gh;
  const int q_tiles = (a.max_seqlen_q + u.tq - 1) / u.tq;
  int L = blockIdx.x;
  const int per_split = q_tiles * a.batch * head_groups;
  u.split = L / per_split;
  L %= per_split;
  int qt;
  if (a.kv_splits > 1) {
    qt = (L / head_groups) % q_tiles;
    u.b = L / (head_groups * q_tiles);
  } else {
    qt = L / (a.batch * head_groups);
    u.b = (L / head_groups) % a.batch;
  }
  u.h0 = (L % head_groups) * u.gh;
  u.kvh = u.h0 / group;
  const int q_lo = a.cu_seqlens_q[u.b];
  u.lq = a.cu_seqlens_q[u.b + 1] - q_lo;
  u.q_off = q_lo;
  if (a.block_table) {
    u.lk = a.seq_lens_kv[u.b];
    u.kv_off = 0;
  } else {
    u.kv_off = a.cu_seqlens_kv[u.b];
    u.lk = a.cu_seqlens_kv[u.b + 1] - (int)u.kv_off;
  }
  u.q_end = u.lq - qt * u.tq;
  u.q_begin = max(0, u.q_end - u.tq);
  return u.q_end > 0;
}

// pf_unit for launches whose per-head K/V fits one XCD's L2 (the FP8 MLA
// prefill: 2.5 MB per head at 8K keys): each XCD walks its own heads HB at a
// time, all query tiles of those heads (longest first) before the next HB,
// so the workgroups running on an XCD share the K/V of HB heads instead of
// one or two tiles of every head (blocks go to the XCDs in turn, so block i
// runs on XCD i % 8). Falls back to pf_unit when the heads or blocks do not
// divide evenly, or with key splits.
template <int HB>
__device__ __forceinline__ bool pf_unit_xcd_heads(const PrefillArgs &a, int blocks, PfUnit &u) {
  constexpr int kXcds = 8;
  const int group = a.num_q_heads / a.num_kv_heads;
  u.gh = pf_heads_per_wg(group);
  u.tq = 32 * (blocks / u.gh);
  const int head_groups = a.num_q_heads / u.gh;
  const int q_tiles = (a.max_seqlen_q + u.tq - 1) / u.tq;
  if (a.kv_splits > 1 || head_groups % (kXcds * HB) != 0) return pf_unit(a, blocks, u);
  const int x = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
  const int per_round = HB * q_tiles * a.batch;          // blocks of one XCD's round of HB heads
  const int round = k / per_round, r = k % per_round;
  const int qt = r / (HB * a.batch), rest = r % (HB * a.batch);
  u.b = rest / HB;
  u.split = 0;
  u.h0 = ((round * kXcds + x) * HB + rest % HB) * u.gh;
  u.kvh = u.h0 / group;
  const int q_lo = a.cu_seqlens_q[u.b];
  u.lq = a.cu_seqlens_q[u.b + 1] - q_lo;
  u.q_off = q_lo;
  if (a.block_table) {
    u.lk = a.seq_lens_kv[u.b];
    u.kv_off = 0;
  } else {
    u.kv_off = a.cu_seqlens_kv[u.b];
    u.lk = a.cu_seqlens_kv[u.b + 1] - (int)u.kv_off;
  }
  u.q_end = u.lq - qt * u.tq;
  u.q_begin = max(0, u.q_end - u.tq);
  return u.q_end > 0;
}

}  // namespace
}  // namespace attn
