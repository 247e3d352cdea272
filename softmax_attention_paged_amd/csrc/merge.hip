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
// weights with wave shuffles. The row's float4 chunks are spread over the
// lanes; when they do not fill the wave, lane groups take every G-th split
// and are summed with shuffles at the end. A lane holding CPL chunks of a
// row reads 16 / CPL partial rows at once, so up to 16 float4 loads per lane
// are in flight together (a 22-split decode of 128-wide rows is read in one
// batch: one round trip for the LSEs, one for the partials). Splits with
// weight 0 (lse = -inf, an empty split) are never read.

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

constexpr int kMergeWaves = 4;
constexpr int kLoadsInFlight = 16;     // float4 loads per lane issued together

// CPL: float4 chunks per lane (1, 2 or 4; head_dim_v <= 1024).
template <int CPL>
__global__ __launch_bounds__(256) void merge_lse_kernel(const MergeArgs a) {
  constexpr int kBatch = kLoadsInFlight / CPL;   // partial rows read together
  const int lane = threadIdx.x & 63;
  const int64_t rowi = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (rowi >= a.num_rows) return;

  // split weights: lane holds splits lane, lane + 64, ...
  float lse_r[kMaxSplits / 64];
  float mmax = kNegInf;
#pragma unroll
  for (int j = 0; j < kMaxSplits / 64; ++j) {
    const int s = lane + 64 * j;
    lse_r[j] = (s < a.num_splits) ? a.lse_parts[(int64_t)s * a.num_rows + rowi] : kNegInf;
    mmax = fmaxf(mmax, lse_r[j]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mmax = fmaxf(mmax, wave_shfl_xor(mmax, off));
  const float muse = (mmax == kNegInf) ? 0.f : mmax;
  float wsum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxSplits / 64; ++j) {
    lse_r[j] = exp2_fast(lse_r[j] - muse);   // weight; 0 for empty splits
    wsum += lse_r[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += wave_shfl_xor(wsum, off);

  // lane layout: G groups of 64 / G lanes; group g sums splits g, g + G, ...
  const int nchunks = a.head_dim_v >> 2;
  const int G = nchunks >= 64 ? 1 : (nchunks >= 32 ? 2 : 4);
  const int glanes = 64 / G;
  const int g = lane / glanes, gl = lane % glanes;
  f32x4 acc[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s0 = 0; s0 < a.num_splits; s0 += kBatch * G) {
    float w[kBatch];
    f32x4 v[kBatch][CPL];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sg = s0 + u * G;            // this batch slot's split for group 0; group g adds g
      float wu = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {         // the weight of split sg + g, from its lane
        const int sq = sg + q;
        const float wq = (sq < a.num_splits) ? __shfl(lse_r[(sq >> 6) & (kMaxSplits / 64 - 1)], sq & 63, 64) : 0.f;
        if (q == g) wu = wq;
      }
      w[u] = wu;
      const int s = sg + g;
      const float *src = a.o_parts + ((int64_t)s * a.num_rows + rowi) * a.head_dim_v;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = gl + glanes * k;
        v[u][k] = (wu != 0.f && c < nchunks) ? *reinterpret_cast<const f32x4 *>(src + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
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
  if (cpl <= 1)
    hipLaunchKernelGGL(merge_lse_kernel<1>, grid, block, 0, stream, a);
  else if (cpl == 2)
    hipLaunchKernelGGL(merge_lse_kernel<2>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(merge_lse_kernel<4>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
