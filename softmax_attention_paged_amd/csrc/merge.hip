// Log-sum-exp merge of split-KV partials, for gfx950.
//
// Split i of a row holds o_i, the output normalised over the split's keys,
// and lse_i = log2 of the split's softmax denominator. The row's output over
// all keys is sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M) with M = max_i
// lse_i, and its log-sum-exp is M + log2(sum_i 2^(lse_i - M)) ("TokenSpeed-
// MLA", section "Decode performance": a second kernel reduces the split-KV
// partial results; section "FP8 split-KV partial storage": combine normalised
// FP32 partials).
//
// One wave per row: the lanes read the split LSEs once and reduce M and the
// weights with wave shuffles; the weights then go through the wave's LDS
// row to the lanes that scale each partial. The row's float4 chunks are
// spread over the lanes; when they do not fill the wave, lane groups take
// every G-th split and are summed with shuffles at the end. A lane holding
// CPL chunks of a row reads 16 / CPL partial rows at once, so up to 16
// float4 loads per lane are in flight together (a 22-split decode of
// 128-wide rows is read in one batch: one round trip for the LSEs, one for
// the partials). Splits with weight 0 (lse = -inf, an empty split) are
// never read.
//
// The GQA decode's key ranges: a row's pieces are the ranges its request
// meets, found from seq_lens as the split kernel cut them (one round trip);
// their first batch of partial rows is read together with their LSEs (one
// more), since only a causal row's last piece can be empty.

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

constexpr int kMergeWaves = 4;
constexpr int kLoadsInFlight = 16;     // float4 loads per lane issued together

// CPL: float4 chunks per lane (1, 2 or 4; head_dim_v <= 1024). kRanges:
// the pieces of the GQA decode's key ranges (partial i of row r of request
// b at slot (g_first + b + i) * q_len * Hq + r, found from seq_lens as the
// split kernel cut the batch); otherwise splits (partial i of row r at
// i * num_rows + r).
template <int CPL, bool kRanges>
__global__ __launch_bounds__(256) void merge_lse_kernel(const MergeArgs a) {
  constexpr int kBatch = kLoadsInFlight / CPL;   // partial rows read together
  constexpr int kMax = kRanges ? kMaxKeyRanges : kMaxSplits;
  const int lane = threadIdx.x & 63;
  const int64_t rowi = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (rowi >= a.num_rows) return;

  int count = a.num_splits;
  int64_t base = rowi, stride = a.num_rows;
  if constexpr (kRanges) {
    const int b = (int)(rowi / a.rows_per_request);
    const int rr = (int)(rowi % a.rows_per_request);
    const BatchTiles bt = batch_tiles(a.seq_lens, a.batch, a.q_len, a.window_left, b, lane);
    const int ranges = min(a.key_ranges, bt.total);
    const int n = gqa_request_tiles(a.seq_lens[b], a.q_len, a.window_left);
    // the ranges holding the request's first and last tile
    const int g_first = (int)(((int64_t)(bt.below + 1) * ranges - 1) / bt.total);
    const int g_last = (int)(((int64_t)(bt.below + n) * ranges - 1) / bt.total);
    if (g_first == g_last) return;            // inside one range: written final by the split kernel
    count = g_last - g_first + 1;
    base = (int64_t)(g_first + b) * a.rows_per_request + rr;
    stride = a.rows_per_request;
  }

  // lane layout: G groups of 64 / G lanes; group g sums splits g, g + G, ...
  const int nchunks = a.head_dim_v >> 2;
  const int G = nchunks >= 64 ? 1 : (nchunks >= 32 ? 2 : 4);
  const int glanes = 64 / G;
  const int g = lane / glanes, gl = lane % glanes;

  // Key ranges: every piece but a causal row's empty last one holds a
  // partial, so the first batch of partial rows is read together with the
  // LSEs (one round trip instead of two); an empty piece's stale row is
  // selected away by its zero weight below.
  f32x4 first[kRanges ? kBatch : 1][CPL];
  if constexpr (kRanges) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sp = u * G + g;
      const float *src = a.o_parts + (base + sp * stride) * a.head_dim_v;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = gl + glanes * k;
        first[u][k] = (sp < count && c < nchunks) ? *reinterpret_cast<const f32x4 *>(src + 4 * c)
                                                  : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // split weights: lane holds splits lane, lane + 64, ...
  float lse_r[kMax / 64];
  float mmax = kNegInf;
#pragma unroll
  for (int j = 0; j < kMax / 64; ++j) {
    const int s = lane + 64 * j;
    lse_r[j] = (s < count) ? a.lse_parts[base + s * stride] : kNegInf;
    mmax = fmaxf(mmax, lse_r[j]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mmax = fmaxf(mmax, wave_shfl_xor(mmax, off));
  const float muse = (mmax == kNegInf) ? 0.f : mmax;
  float wsum = 0.f;
#pragma unroll
  for (int j = 0; j < kMax / 64; ++j) {
    lse_r[j] = exp2_fast(lse_r[j] - muse);   // weight; 0 for empty splits
    wsum += lse_r[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += wave_shfl_xor(wsum, off);

  f32x4 acc[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The weights go to the wave's LDS row, where each lane group reads those
  // of its splits (LDS operations of one wave execute in order).
  __shared__ float wts[kMergeWaves][kMax];
  float *wrow = wts[threadIdx.x >> 6];
#pragma unroll
  for (int j = 0; j < kMax / 64; ++j) wrow[lane + 64 * j] = lse_r[j];
  asm volatile("" ::: "memory");
  // the weight of split sg + g of this lane's group
  auto weight = [&](int sg) { return (sg + g < count) ? wrow[sg + g] : 0.f; };
  int s_begin = 0;
  if constexpr (kRanges) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float wu = weight(u * G);
#pragma unroll
      for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k][e] += (wu != 0.f) ? wu * first[u][k][e] : 0.f;
    }
    s_begin = kBatch * G;
  }
  for (int s0 = s_begin; s0 < count; s0 += kBatch * G) {
    float w[kBatch];
    f32x4 v[kBatch][CPL];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sg = s0 + u * G;            // this batch slot's split for group 0; group g adds g
      const float wu = weight(sg);
      w[u] = wu;
      const int s = sg + g;
      const float *src = a.o_parts + (base + s * stride) * a.head_dim_v;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = gl + glanes * k;
        v[u][k] = (wu != 0.f && c < nchunks) ? *reinterpret_cast<const f32x4 *>(src + 4 * c)
                                             : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int k = 0; k < CPL; ++k) acc[k] += w[u] * v[u][k];
  }
  // sum the lane groups (lanes gl, gl + glanes, ... hold the same chunks)
  for (int off = glanes; off < 64; off <<= 1)
#pragma unroll
    for (int k = 0; k < CPL; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[k][e] += wave_shfl_xor(acc[k][e], off);

  const float inv = (wsum > 0.f) ? 1.f / wsum : 0.f;
  if (g == 0) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = gl + glanes * k;
      if (c >= nchunks) continue;
      const f32x4 r = acc[k] * inv;
      if (a.o_bf16) {
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = to_bf16(r[e]);
        *reinterpret_cast<u32x2 *>(static_cast<__bf16 *>(a.o) + rowi * a.head_dim_v + 4 * c) =
            __builtin_bit_cast(u32x2, ob);
      } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(a.o) + rowi * a.head_dim_v + 4 * c) = r;
      }
    }
  }
  if (a.lse && lane == 0) a.lse[rowi] = (wsum > 0.f) ? muse + __log2f(wsum) : kNegInf;
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream) {
  const int64_t blocks = (a.num_rows + kMergeWaves - 1) / kMergeWaves;
  // the kernel's lane layout: G groups of 64 / G lanes over the row's chunks
  const int nchunks = a.head_dim_v >> 2;
  const int glanes = 64 / (nchunks >= 64 ? 1 : (nchunks >= 32 ? 2 : 4));
  const int cpl = (nchunks + glanes - 1) / glanes;
  const dim3 grid((unsigned)blocks), block(64 * kMergeWaves);
  if (a.key_ranges > 0) {
    if (cpl <= 1)
      hipLaunchKernelGGL((merge_lse_kernel<1, true>), grid, block, 0, stream, a);
    else if (cpl == 2)
      hipLaunchKernelGGL((merge_lse_kernel<2, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((merge_lse_kernel<4, true>), grid, block, 0, stream, a);
  } else if (cpl <= 1) {
    hipLaunchKernelGGL((merge_lse_kernel<1, false>), grid, block, 0, stream, a);
  } else if (cpl == 2) {
    hipLaunchKernelGGL((merge_lse_kernel<2, false>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((merge_lse_kernel<4, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn
