// Paged GQA decode, split over the KV sequence, for gfx950.
//
// One workgroup = one (request b, KV head, query group, KV split) unit: the
// G query heads that share the KV head ("Writing Page Attention with PyPTO",
// section 1.3: one task is one batch row + one KV head + its query heads,
// so the KV pages are read once for all of them) times the F query tokens
// folded with them into the MFMA row dimension ("TokenSpeed-MLA", section
// "Key Optimization ... Group q_seqlen and num_heads into BMM1 M").
//
// Inside the workgroup, 4 waves take 32-key tiles of the split in turn. Each
// wave keeps its own running max m, sum l and output o per row (the online
// recurrence of "Flywheel Attention", section 1, and "Writing Page Attention
// with PyPTO", section 6.3) and the waves are combined by log-sum-exp at the
// end. Per tile:
//   - K rows are gathered through the block table straight into registers,
//     already in the MFMA A-operand layout (token = l % 16, 8 channels per
//     lane); the page of a 16-key tile is one table entry (pages hold a
//     power of two >= 16 keys), read once per tile.
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
// With one split the workgroup writes bf16 O and the base-2 LSE; otherwise it
// writes FP32 partials (O normalised over the split, LSE of the split) that
// the merge kernel reduces ("TokenSpeed-MLA", section "Decode performance").

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

template <int D>
struct GqaGeom {
  static constexpr int kWaves = kGqaWaves;
  static constexpr int kTile = kGqaTileTokens;                 // 32 keys per wave step
  static constexpr int kKB = D / 32;                            // QK k-steps
  static constexpr int kNB = D / 16;                            // PV 16-channel blocks
  static constexpr int kVStride = D + 16;                       // LDS row stride (bf16), breaks bank aliasing
  static constexpr int kVTile = kTile * kVStride;               // bf16 elements per wave
  static constexpr int kChunksPerRow = D / 8;                   // 16-byte chunks per V row
  static constexpr int kVChunks = kTile * kChunksPerRow / 64;   // 16-byte chunks per lane per V tile
  static constexpr int kLdsV = kWaves * kVTile * 2;
  static constexpr int kLdsMerge = kWaves * 16 * 4 * 3 + kWaves * 16 * D * 4;
  static constexpr int kLds = kLdsV > kLdsMerge ? kLdsV : kLdsMerge;
#ifndef ATTN_DECODE_PREFETCH
#define ATTN_DECODE_PREFETCH 0
#endif
  // Register double-buffering of the next tile (costs ~64 VGPRs at D = 128).
  static constexpr bool kPrefetch = ATTN_DECODE_PREFETCH && D <= 128;
};

template <int D>
struct KvRegs {
  bf16x8 k[2][GqaGeom<D>::kKB];
  bf16x8 v[GqaGeom<D>::kVChunks];
};

template <int D>
__device__ __forceinline__ void load_tile(const DecodeGqaArgs &a, const int32_t *bt_row,
                                          const __bf16 *kbase, const __bf16 *vbase, int tok0,
                                          int end, int lane, KvRegs<D> &r) {
  using G = GqaGeom<D>;
  const int pmask = (1 << a.page_shift) - 1;
  // One table entry per 16-key half-tile; never past the request's pages.
  const int64_t page0 = bt_row[tok0 >> a.page_shift];
  const int64_t page1 = (tok0 + 16 < end) ? (int64_t)bt_row[(tok0 + 16) >> a.page_shift] : page0;
  const int kg = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = tok0 + 16 * t + (lane & 15);
    const int64_t page = t ? page1 : page0;
    const __bf16 *row = kbase + page * a.k_stride_page + (int64_t)(tok & pmask) * a.k_stride_tok;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb) r.k[t][kb] = load_bf16x8(row + kb * 32 + kg * 8);
  }
#pragma unroll
  for (int c = 0; c < G::kVChunks; ++c) {
    const int idx = c * 64 + lane;
    const int trow = idx / G::kChunksPerRow;          // 0..31
    const int col = (idx % G::kChunksPerRow) * 8;
    const int tok = tok0 + trow;
    const int64_t page = (trow >= 16) ? page1 : page0;
    const __bf16 *row = vbase + page * a.v_stride_page + (int64_t)(tok & pmask) * a.v_stride_tok;
    bf16x8 v = load_bf16x8(row + col);
    r.v[c] = (tok < end) ? v : bf16x8{};
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void decode_gqa_kernel(const DecodeGqaArgs a) {
  using G = GqaGeom<D>;
  __shared__ __attribute__((aligned(16))) char smem[G::kLds];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kg = lane >> 4;          // lane group 0..3
  const int row = lane & 15;         // the score/output row this lane owns

  // unit -> (b, kv head, q group, split)
  int unit = blockIdx.x;
  const int split = unit % a.num_splits;
  unit /= a.num_splits;
  const int qg = unit % a.q_groups;
  unit /= a.q_groups;
  const int kvh = unit % a.num_kv_heads;
  const int b = unit / a.num_kv_heads;

  const int lk = a.seq_lens[b];
  // Row r of the unit is query token qg*F + r/G, head kvh*G + r%G.
  const bool row_valid = row < a.rows;
  const int t_row = qg * a.fold + (row_valid ? row / a.group : 0);
  const int h_row = kvh * a.group + (row_valid ? row % a.group : 0);
  int bound = lk;
  if (a.causal) bound = min(lk, max(0, lk - a.q_len + t_row + 1));
  // keys any row of the unit may see (the last folded token sees the most)
  int unit_bound = lk;
  if (a.causal) unit_bound = min(lk, max(0, lk - a.q_len + qg * a.fold + a.fold));

  const int c0 = split * a.split_tokens;
  const int c1 = min(unit_bound, c0 + a.split_tokens);
  const int row_end = min(bound, c1);
  const int64_t R = (int64_t)a.batch * a.q_len * a.num_q_heads;
  const int64_t ridx = ((int64_t)b * a.q_len + t_row) * a.num_q_heads + h_row;

  if (c0 >= c1) {
    // Nothing to attend to in this split.
    if (threadIdx.x < 64 && kg == 0 && row_valid) {
      if (a.num_splits == 1) {
        if (a.lse) a.lse[ridx] = kNegInf;
      } else {
        a.lse_parts[(int64_t)split * R + ridx] = kNegInf;
      }
    }
    if (a.num_splits == 1) {
      // rows without keys: O = 0
      for (int ch = threadIdx.x; ch < 16 * G::kChunksPerRow; ch += 256) {
        const int r = ch / G::kChunksPerRow;
        if (r >= a.rows) continue;
        const int t = qg * a.fold + r / a.group;
        const int h = kvh * a.group + r % a.group;
        const int64_t ri = ((int64_t)b * a.q_len + t) * a.num_q_heads + h;
        *reinterpret_cast<u32x4 *>(static_cast<__bf16 *>(a.o) + ri * D + (ch % G::kChunksPerRow) * 8) = u32x4{};
      }
    }
    return;
  }

  // Q^T as the MFMA B operand: row l%16, channels 32kb + 8kg + e.
  bf16x8 qop[G::kKB];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + ridx * D;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
      qop[kb] = row_valid ? load_bf16x8(qrow + kb * 32 + kg * 8) : bf16x8{};
  }

  const int32_t *bt_row = a.block_table + (int64_t)b * a.block_table_stride;
  const __bf16 *kbase = static_cast<const __bf16 *>(a.k_cache) + (int64_t)kvh * a.k_stride_head;
  const __bf16 *vbase = static_cast<const __bf16 *>(a.v_cache) + (int64_t)kvh * a.v_stride_head;
  __bf16 *vlds = reinterpret_cast<__bf16 *>(smem) + wave * G::kVTile;

  float m = kNegInf;   // running max, log2 units of the scaled score
  float lsum = 0.f;    // running sum of bf16-rounded p over this lane's keys
  float lexact = 0.f;  // running sum of fp32 p over this lane's keys
  f32x4 oacc[G::kNB];
#pragma unroll
  for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int tok0, const KvRegs<D> &r) {
    // S^T tiles: acc[0] keys tok0 + 4kg + i, acc[1] keys tok0 + 16 + 4kg + i.
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb) sacc[t] = mfma16x16x32(r.k[t][kb], qop[kb], sacc[t]);
    }
    // V tile -> LDS (token-major), for the transposing read.
#pragma unroll
    for (int c = 0; c < G::kVChunks; ++c) {
      const int idx = c * 64 + lane;
      const int trow = idx / G::kChunksPerRow;
      const int col = (idx % G::kChunksPerRow) * 8;
      store_bf16x8_lds(vlds + trow * G::kVStride + col, r.v[c]);
    }
    float x[8];
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tok0 + 16 * t + 4 * kg + i;
        const float v = (j < row_end) ? sacc[t][i] * a.scale_log2 : kNegInf;
        x[4 * t + i] = v;
        mx = fmaxf(mx, v);
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
    // O^T[16 channels x 16 rows] += V^T[channels x 32 keys] * P^T[32 keys x rows]
    // k-slot e of lane group kg is key 4kg + e (e < 4) or 16 + 4kg + e - 4.
    const int src_row = 4 * kg + (row >> 2);
    const int src_col = 4 * (row & 3);
#pragma unroll
    for (int nb = 0; nb < G::kNB; ++nb) {
      const bf16x4 lo = lds_read_tr16(vlds + src_row * G::kVStride + nb * 16 + src_col);
      const bf16x4 hi = lds_read_tr16(vlds + (16 + src_row) * G::kVStride + nb * 16 + src_col);
      oacc[nb] = mfma16x16x32(concat(lo, hi), pop, oacc[nb]);
    }
  };

  // Two register buffers: the next tile's loads are in flight while the
  // current one is computed.
  const int step = G::kWaves * G::kTile;
  int tok0 = c0 + wave * G::kTile;
  if constexpr (G::kPrefetch) {
    KvRegs<D> ra, rb;
    if (tok0 < c1) load_tile<D>(a, bt_row, kbase, vbase, tok0, c1, lane, ra);
    while (tok0 < c1) {
      if (tok0 + step < c1) load_tile<D>(a, bt_row, kbase, vbase, tok0 + step, c1, lane, rb);
      compute(tok0, ra);
      tok0 += step;
      if (tok0 >= c1) break;
      if (tok0 + step < c1) load_tile<D>(a, bt_row, kbase, vbase, tok0 + step, c1, lane, ra);
      compute(tok0, rb);
      tok0 += step;
    }
  } else {
    for (; tok0 < c1; tok0 += step) {
      KvRegs<D> cur;
      load_tile<D>(a, bt_row, kbase, vbase, tok0, c1, lane, cur);
      compute(tok0, cur);
    }
  }

  // ---- combine the 4 waves by log-sum-exp ----
  lsum += wave_shfl_xor(lsum, 16);
  lsum += wave_shfl_xor(lsum, 32);
  lexact += wave_shfl_xor(lexact, 16);
  lexact += wave_shfl_xor(lexact, 32);
  __syncthreads();  // every wave is done with its V tile region
  float *sm_m = reinterpret_cast<float *>(smem);
  float *sm_l = sm_m + G::kWaves * 16;
  float *sm_le = sm_l + G::kWaves * 16;
  float *sm_o = sm_le + G::kWaves * 16;
  if (kg == 0) {
    sm_m[wave * 16 + row] = m;
    sm_l[wave * 16 + row] = lsum;
    sm_le[wave * 16 + row] = lexact;
  }
#pragma unroll
  for (int nb = 0; nb < G::kNB; ++nb)
    *reinterpret_cast<f32x4 *>(sm_o + (wave * 16 + row) * D + nb * 16 + 4 * kg) = oacc[nb];
  __syncthreads();

  for (int ch = threadIdx.x; ch < 16 * G::kChunksPerRow; ch += 256) {
    const int r = ch / G::kChunksPerRow;
    if (r >= a.rows) continue;
    const int c8 = (ch % G::kChunksPerRow) * 8;
    float mw[G::kWaves];
    float mmax = kNegInf;
#pragma unroll
    for (int w = 0; w < G::kWaves; ++w) {
      mw[w] = sm_m[w * 16 + r];
      mmax = fmaxf(mmax, mw[w]);
    }
    const float muse = (mmax == kNegInf) ? 0.f : mmax;
    float f[G::kWaves];
    float L = 0.f, Le = 0.f;
#pragma unroll
    for (int w = 0; w < G::kWaves; ++w) {
      f[w] = exp2_fast(mw[w] - muse);
      L += f[w] * sm_l[w * 16 + r];
      Le += f[w] * sm_le[w * 16 + r];
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = 0.f;
#pragma unroll
    for (int w = 0; w < G::kWaves; ++w) {
      const f32x4 lo = *reinterpret_cast<const f32x4 *>(sm_o + (w * 16 + r) * D + c8);
      const f32x4 hi = *reinterpret_cast<const f32x4 *>(sm_o + (w * 16 + r) * D + c8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[e] += f[w] * lo[e];
        out[4 + e] += f[w] * hi[e];
      }
    }
    const int t = qg * a.fold + r / a.group;
    const int h = kvh * a.group + r % a.group;
    const int64_t ri = ((int64_t)b * a.q_len + t) * a.num_q_heads + h;
    const float lse2 = (Le > 0.f) ? muse + __log2f(Le) : kNegInf;
    if (a.num_splits == 1) {
      bf16x8 ob;
#pragma unroll
      for (int e = 0; e < 8; ++e) ob[e] = to_bf16(out[e] * inv);
      *reinterpret_cast<u32x4 *>(static_cast<__bf16 *>(a.o) + ri * D + c8) = __builtin_bit_cast(u32x4, ob);
      if (a.lse && c8 == 0) a.lse[ri] = lse2;
    } else {
      float *dst = a.o_parts + ((int64_t)split * R + ri) * D + c8;
      *reinterpret_cast<f32x4 *>(dst) = f32x4{out[0] * inv, out[1] * inv, out[2] * inv, out[3] * inv};
      *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{out[4] * inv, out[5] * inv, out[6] * inv, out[7] * inv};
      if (c8 == 0) a.lse_parts[(int64_t)split * R + ri] = lse2;
    }
  }
}

}  // namespace

hipError_t launch_decode_gqa(const DecodeGqaArgs &a, hipStream_t stream) {
  const int64_t units = (int64_t)a.batch * a.num_kv_heads * a.q_groups * a.num_splits;
  const dim3 grid((unsigned)units), block(256);
  switch (a.head_dim) {
    case 64: hipLaunchKernelGGL(decode_gqa_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(decode_gqa_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(decode_gqa_kernel<256>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
