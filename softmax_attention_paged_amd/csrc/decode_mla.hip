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
// Workgroup: 8 waves x 16 rows. Per 32-key tile:
//   - the latent tile is gathered through the block table and stored ONCE
//     in LDS (double-buffered, loaded one tile ahead through registers): the
//     same bytes serve as K and as V;
//   - FP8 e4m3 codes are widened to bf16 exactly while staging (every e4m3
//     value is a bf16 value) and the per-tensor scale is applied to the
//     scores and to the final output instead ("TokenSpeed-MLA": FP8 KV with
//     FP32 softmax exponentials and sums, bf16 output);
//   - S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with the
//     row state lane-local as in the GQA decode kernel; V^T is read from LDS
//     with ds_read_b64_tr_b16.
// Workgroups are renumbered so that consecutive units run on the same XCD:
// the query groups of one split then share that XCD's L2 for the latent.

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

constexpr int kDk = 576;
constexpr int kDv = 512;
constexpr int kMlaWaves = 8;
constexpr int kTileN = kMlaTileTokens;            // 32 keys per tile
constexpr int kStride = kDk + 16;                 // LDS row stride (bf16)
constexpr int kTileElems = kTileN * kStride;
constexpr int kKB = kDk / 32;                     // 18 QK k-steps
constexpr int kNB = kDv / 16;                     // 32 PV channel blocks
constexpr int kThreads = 64 * kMlaWaves;
constexpr int kXcds = 8;

// Chunks a thread stages per tile: bf16 rows are 72 16-byte chunks, fp8 rows 36.
template <bool FP8>
struct Stage {
  static constexpr int kRowChunks = FP8 ? kDk / 16 : kDk / 8;
  static constexpr int kChunks = kTileN * kRowChunks;
  static constexpr int kPerThread = (kChunks + kThreads - 1) / kThreads;
};

// Bijective renumbering: hardware dispatches workgroup i to XCD i % 8; unit
// numbers handed to one XCD become consecutive.
__device__ __forceinline__ int xcd_unit(int i, int n) {
  const int per = n / kXcds, rem = n % kXcds;
  const int x = i % kXcds, k = i / kXcds;
  return x * per + min(x, rem) + k;
}

// Exact e4m3 -> bf16 of 16 codes (the hardware FP8 convert reads the OCP format on gfx950).
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 w, bf16x8 &lo, bf16x8 &hi) {
  float f[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int word = (int)w[q];
    const auto p01 = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);   // bytes 0, 1
    const auto p23 = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);    // bytes 2, 3
    f[4 * q + 0] = p01[0];
    f[4 * q + 1] = p01[1];
    f[4 * q + 2] = p23[0];
    f[4 * q + 3] = p23[1];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = to_bf16(f[e]);
    hi[e] = to_bf16(f[8 + e]);
  }
}

template <bool FP8>
__device__ __forceinline__ void stage_load(const DecodeMlaArgs &a, const int32_t *bt_row, int j0, int end, int tid,
                                           u32x4 (&r)[Stage<FP8>::kPerThread]) {
  using S = Stage<FP8>;
  const int pmask = (1 << a.page_shift) - 1;
#pragma unroll
  for (int c = 0; c < S::kPerThread; ++c) {
    const int idx = c * kThreads + tid;
    const int trow = idx / S::kRowChunks;
    const int j = j0 + trow;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (idx < S::kChunks && j < end) {
      const int64_t page = bt_row[j >> a.page_shift];
      const int64_t elem = page * a.kv_stride_page + (int64_t)(j & pmask) * a.kv_stride_tok +
                           (idx % S::kRowChunks) * (FP8 ? 16 : 8);
      const char *base = static_cast<const char *>(a.kv_cache) + elem * (FP8 ? 1 : 2);
      v = *reinterpret_cast<const u32x4 *>(base);
    }
    r[c] = v;
  }
}

template <bool FP8>
__device__ __forceinline__ void stage_store(__bf16 *tile, int tid, const u32x4 (&r)[Stage<FP8>::kPerThread]) {
  using S = Stage<FP8>;
#pragma unroll
  for (int c = 0; c < S::kPerThread; ++c) {
    const int idx = c * kThreads + tid;
    if (idx >= S::kChunks) continue;
    const int trow = idx / S::kRowChunks;
    if constexpr (FP8) {
      bf16x8 lo, hi;
      fp8x16_to_bf16(r[c], lo, hi);
      __bf16 *dst = tile + trow * kStride + (idx % S::kRowChunks) * 16;
      store_bf16x8_lds(dst, lo);
      store_bf16x8_lds(dst + 8, hi);
    } else {
      store_bf16x8_lds(tile + trow * kStride + (idx % S::kRowChunks) * 8, __builtin_bit_cast(bf16x8, r[c]));
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void decode_mla_kernel(const DecodeMlaArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 tiles[2 * kTileElems];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 4;
  const int row16 = lane & 15;

  const int n_units = a.batch * a.num_splits * a.q_groups;
  int unit = xcd_unit(blockIdx.x, n_units);
  const int qg = unit % a.q_groups;
  unit /= a.q_groups;
  const int split = unit % a.num_splits;
  const int b = unit / a.num_splits;

  const int lk = a.seq_lens[b];
  int unit_bound = lk;
  if (a.causal) unit_bound = min(lk, max(0, lk - a.q_len + qg * a.fold + a.fold));
  const int c0 = split * a.split_tokens;
  const int c1 = min(unit_bound, c0 + a.split_tokens);

  // this lane's row: r = 16 * wave + lane % 16 -> query token qg*F + r/H, head r%H
  const int r = 16 * wave + row16;
  const bool row_valid = r < a.rows;
  const int t_row = qg * a.fold + (row_valid ? r / a.num_heads : 0);
  const int h_row = row_valid ? r % a.num_heads : 0;
  const int64_t R = (int64_t)a.batch * a.q_len * a.num_heads;
  const int64_t ridx = ((int64_t)b * a.q_len + t_row) * a.num_heads + h_row;
  int bound = lk;
  if (a.causal) bound = min(lk, max(0, lk - a.q_len + t_row + 1));
  const int row_end = min(bound, c1);
  const bool wave_active = 16 * wave < a.rows;

  if (c0 >= c1) {   // uniform: no key of this split is visible
    if (row_valid) {
      if (a.num_splits == 1) {
        __bf16 *dst = static_cast<__bf16 *>(a.o) + ridx * kDv + 4 * kg;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) *reinterpret_cast<u32x2 *>(dst + nb * 16) = u32x2{0u, 0u};
        if (a.lse && kg == 0) a.lse[ridx] = kNegInf;
      } else if (kg == 0) {
        a.lse_parts[(int64_t)split * R + ridx] = kNegInf;
      }
    }
    return;
  }

  // Q^T operand: lane holds Q[row r][32kb + 8kg .. +8]
  bf16x8 qop[kKB];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + ridx * kDk;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) qop[kb] = row_valid ? load_bf16x8(qrow + kb * 32 + kg * 8) : bf16x8{};
  }
  float m = kNegInf, lsum = 0.f, lexact = 0.f;
  f32x4 oacc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t *bt_row = a.block_table + (int64_t)b * a.block_table_stride;
  u32x4 stage[Stage<FP8>::kPerThread];
  stage_load<FP8>(a, bt_row, c0, c1, tid, stage);
  stage_store<FP8>(tiles, tid, stage);
  __syncthreads();

  const int ntiles = (c1 - c0 + kTileN - 1) / kTileN;
  const int src_row = 4 * kg + (row16 >> 2);
  const int src_col = 4 * (row16 & 3);
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = c0 + it * kTileN;
    const __bf16 *tile = tiles + (it & 1) * kTileElems;
    const bool more = it + 1 < ntiles;
    if (more) stage_load<FP8>(a, bt_row, j0 + kTileN, c1, tid, stage);

    if (wave_active) {
      // S^T: sacc[t] holds keys j0 + 16t + 4kg + i of row r
      f32x4 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const __bf16 *krow = tile + (16 * t + row16) * kStride + 8 * kg;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
          sacc[t] = mfma16x16x32(*reinterpret_cast<const bf16x8 *>(krow + 32 * kb), qop[kb], sacc[t]);
      }
      float x[8];
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 16 * t + 4 * kg + i;
          const float v = (j < row_end) ? sacc[t][i] * a.scale_log2 : kNegInf;
          x[4 * t + i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, wave_shfl_xor(mx, 16));
      mx = fmaxf(mx, wave_shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      m = m_new;
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
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) oacc[nb] *= alpha;
      // O^T += V^T P^T; V is the first 512 columns of the latent tile
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const bf16x4 lo = lds_read_tr16(tile + src_row * kStride + nb * 16 + src_col);
        const bf16x4 hi = lds_read_tr16(tile + (16 + src_row) * kStride + nb * 16 + src_col);
        oacc[nb] = mfma16x16x32(concat(lo, hi), pop, oacc[nb]);
      }
    }

    if (more) stage_store<FP8>(tiles + ((it + 1) & 1) * kTileElems, tid, stage);
    __syncthreads();
  }

  // ---- epilogue: each wave writes its own rows ----
  lsum += wave_shfl_xor(lsum, 16);
  lsum += wave_shfl_xor(lsum, 32);
  lexact += wave_shfl_xor(lexact, 16);
  lexact += wave_shfl_xor(lexact, 32);
  if (!row_valid) return;
  const float inv = (lsum > 0.f) ? a.kv_scale / lsum : 0.f;     // V dequantisation folded in
  const float muse = (m == kNegInf) ? 0.f : m;
  const float lse2 = (lexact > 0.f) ? muse + __log2f(lexact) : kNegInf;
  if (a.num_splits == 1) {
    __bf16 *dst = static_cast<__bf16 *>(a.o) + ridx * kDv + 4 * kg;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      bf16x4 ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) ob[i] = to_bf16(oacc[nb][i] * inv);
      *reinterpret_cast<u32x2 *>(dst + nb * 16) = __builtin_bit_cast(u32x2, ob);
    }
    if (a.lse && kg == 0) a.lse[ridx] = lse2;
  } else {
    float *dst = a.o_parts + ((int64_t)split * R + ridx) * kDv + 4 * kg;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) *reinterpret_cast<f32x4 *>(dst + nb * 16) = oacc[nb] * inv;
    if (kg == 0) a.lse_parts[(int64_t)split * R + ridx] = lse2;
  }
}

}  // namespace

hipError_t launch_decode_mla(const DecodeMlaArgs &a, hipStream_t stream) {
  const int64_t units = (int64_t)a.batch * a.num_splits * a.q_groups;
  if (a.kv_fp8)
    hipLaunchKernelGGL(decode_mla_kernel<true>, dim3((unsigned)units), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_mla_kernel<false>, dim3((unsigned)units), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
