// Ragged prefill over dense or paged KV, causal (bottom-right) or not, for gfx950.
//
// Computes, for every query row of every head, softmax attention over the
// keys the row may see, with the running-max / running-sum recurrence over
// key tiles ("Flywheel Attention: Attention Kernels Built for the TPU",
// section 1; "Writing Page Attention with PyPTO", section 6.3), and the
// base-2 log-sum-exp ("TokenSpeed-MLA", kernel capability summary: optional
// FP32 LSE, base-2 semantics).
//
// Workgroup = 4 waves = 128 query rows that share one KV head: GH query heads
// of a GQA group (GH in {1, 2, 4}) times 128 / GH consecutive query tokens.
// Wave w owns 32 rows: tokens of one head. Per 64-key tile (32 at D = 256):
//   - the tile's K and V rows are gathered (through the block table when
//     paged, "Writing Page Attention with PyPTO", section 5.2) with 16-byte
//     loads into registers one tile ahead, then stored to a double-buffered,
//     padded LDS tile; keys past the request are zeroed, table entries past
//     its last page are never read (section 9);
//   - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with Q^T held in registers, so
//     each lane holds 16 scores of one row per 32 keys;
//   - masking (tail, and above the bottom-right causal diagonal) only on the
//     tiles that reach a row bound; masked scores are -inf before the max;
//   - P rounded to bf16 (RNE) is the B operand of O^T += V^T P^T straight
//     from the score registers; V^T comes from LDS via ds_read_b64_tr_b16.
// The rounded P sums normalise O, the FP32 P sums give the LSE. Query tiles
// are aligned to the END of each request, so tile 0 of every request sees
// the most keys and is launched first.

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfRows = 32;                  // rows per wave
constexpr int kPfBlockRows = kPfWaves * kPfRows;

template <int D>
struct PfGeom {
  static constexpr int kN = D <= 128 ? 64 : 32;       // keys per tile
  static constexpr int kSub = kN / 32;                // 32-key S^T sub-tiles
  static constexpr int kKB = D / 16;                  // QK k-steps (16 channels)
  static constexpr int kNB = D / 32;                  // PV 32-channel blocks
  static constexpr int kStride = D + 16;              // LDS row stride (bf16)
  static constexpr int kTileElems = kN * kStride;
  static constexpr int kChunksPerRow = D / 8;         // 16-byte chunks per row
  static constexpr int kChunks = kN * kChunksPerRow / (64 * kPfWaves);  // per thread, per tensor
  static constexpr int kLds = 2 /*K,V*/ * 2 /*buffers*/ * kTileElems * 2;
};

struct PfUnit {
  int b, kvh, h0, gh;          // request, KV head, first query head, heads per workgroup
  int q_begin, q_end;          // query rows of the request covered by this workgroup (relative)
  int lq, lk;                  // request lengths
  int64_t q_off;               // first query token of the request in the packed Q
  int64_t kv_off;              // dense: first key of the request in packed K/V
};

template <int D>
struct PfTileRegs {
  bf16x8 k[PfGeom<D>::kChunks];
  bf16x8 v[PfGeom<D>::kChunks];
};

template <int D>
__device__ __forceinline__ void pf_load_tile(const PrefillArgs &a, const PfUnit &u, int j0, int tid,
                                             PfTileRegs<D> &r) {
  using G = PfGeom<D>;
  const int32_t *bt_row = a.block_table ? a.block_table + (int64_t)u.b * a.block_table_stride : nullptr;
  const int pmask = (1 << a.page_shift) - 1;
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    const int idx = c * 64 * kPfWaves + tid;
    const int trow = idx / G::kChunksPerRow;
    const int col = (idx % G::kChunksPerRow) * 8;
    const int j = j0 + trow;
    bf16x8 kv = bf16x8{}, vv = bf16x8{};
    if (j < u.lk) {
      const __bf16 *kp, *vp;
      if (bt_row) {
        const int64_t page = bt_row[j >> a.page_shift];
        const int64_t slot = j & pmask;
        kp = static_cast<const __bf16 *>(a.k) + page * a.k_stride_page + slot * a.k_stride_tok;
        vp = static_cast<const __bf16 *>(a.v) + page * a.v_stride_page + slot * a.v_stride_tok;
      } else {
        kp = static_cast<const __bf16 *>(a.k) + (u.kv_off + j) * a.k_stride_tok;
        vp = static_cast<const __bf16 *>(a.v) + (u.kv_off + j) * a.v_stride_tok;
      }
      kv = load_bf16x8(kp + (int64_t)u.kvh * a.k_stride_head + col);
      vv = load_bf16x8(vp + (int64_t)u.kvh * a.v_stride_head + col);
    }
    r.k[c] = kv;
    r.v[c] = vv;
  }
}

template <int D>
__device__ __forceinline__ void pf_store_tile(__bf16 *klds, __bf16 *vlds, int tid, const PfTileRegs<D> &r) {
  using G = PfGeom<D>;
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    const int idx = c * 64 * kPfWaves + tid;
    const int off = (idx / G::kChunksPerRow) * G::kStride + (idx % G::kChunksPerRow) * 8;
    store_bf16x8_lds(klds + off, r.k[c]);
    store_bf16x8_lds(vlds + off, r.v[c]);
  }
}

template <int D>
__global__ __launch_bounds__(64 * kPfWaves) void prefill_kernel(const PrefillArgs a) {
  using G = PfGeom<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[G::kLds / 2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;           // lane half
  const int r32 = lane & 31;         // this lane's row within the wave

  // ---- which rows this workgroup owns ----
  const int group = a.num_q_heads / a.num_kv_heads;
  const int gh = (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
  const int tq = kPfBlockRows / gh;                 // query tokens per workgroup
  const int head_groups = a.num_q_heads / gh;
  int L = blockIdx.x;
  const int qt = L / (a.batch * head_groups);       // tile index counted from the request's end
  L %= a.batch * head_groups;
  const int hg = L % head_groups;
  PfUnit u;
  u.b = L / head_groups;
  u.gh = gh;
  u.h0 = hg * gh;
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
  u.q_end = u.lq - qt * tq;
  u.q_begin = max(0, u.q_end - tq);
  if (u.q_end <= 0) return;          // uniform: this request has fewer tiles

  // ---- this wave's 32 rows: head h0 + w / (4/gh), tokens of block w % (4/gh) ----
  const int waves_per_head = kPfWaves / gh;
  const int head = u.h0 + wave / waves_per_head;
  const int tok_base = u.q_end - tq + (wave % waves_per_head) * kPfRows;   // may be < 0 at the top
  const int t = tok_base + r32;                                            // this lane's query row
  const bool row_valid = t >= u.q_begin && t < u.q_end;
  // keys row t sees: [0, bound)
  int bound = u.lk;
  if (a.causal) bound = min(u.lk, max(0, u.lk - u.lq + t + 1));
  if (!row_valid) bound = 0;
  // keys the workgroup must walk, and where this wave's masking starts
  int kv_end = u.lk;
  if (a.causal) kv_end = min(u.lk, max(0, u.lk - u.lq + u.q_end));
  int wave_min = bound, wave_max = bound;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    wave_min = min(wave_min, __shfl_xor(wave_min, off, 64));
    wave_max = max(wave_max, __shfl_xor(wave_max, off, 64));
  }
  // lanes of invalid rows pull wave_min to 0; mask from the smallest valid bound instead
  int valid_min = row_valid ? bound : 0x7fffffff;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) valid_min = min(valid_min, __shfl_xor(valid_min, off, 64));
  (void)wave_min;

  // ---- Q^T operand: lane holds Q[row t][16kb + 8h .. +8] ----
  bf16x8 qop[G::kKB];
  {
    const __bf16 *qrow = static_cast<const __bf16 *>(a.q) + (u.q_off + t) * a.q_stride_tok + (int64_t)head * a.q_stride_head;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb) qop[kb] = row_valid ? load_bf16x8(qrow + kb * 16 + h * 8) : bf16x8{};
  }

  float m = kNegInf, lsum = 0.f, lexact = 0.f;
  f32x16 oacc[G::kNB];
#pragma unroll
  for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] = f32x16{};

  const int ntiles = (kv_end + G::kN - 1) / G::kN;
  PfTileRegs<D> regs;
  if (ntiles > 0) {
    pf_load_tile<D>(a, u, 0, tid, regs);
    pf_store_tile<D>(lds, lds + G::kTileElems, tid, regs);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int j0 = it * G::kN;
    const __bf16 *klds = lds + (it & 1) * 2 * G::kTileElems;
    const __bf16 *vlds = klds + G::kTileElems;
    const bool more = it + 1 < ntiles;
    if (more) pf_load_tile<D>(a, u, j0 + G::kN, tid, regs);

    if (j0 < wave_max) {
      // ---- S^T = K Q^T, kSub sub-tiles of 32 keys ----
      f32x16 sacc[G::kSub];
#pragma unroll
      for (int s = 0; s < G::kSub; ++s) {
        sacc[s] = f32x16{};
        const __bf16 *krow = klds + (32 * s + r32) * G::kStride + h * 8;
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb) {
          const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(krow + kb * 16);
          sacc[s] = mfma32x32x16(kop, qop[kb], sacc[s]);
        }
      }
      // ---- scale, mask, online softmax (row r32 lives in this lane) ----
      const bool need_mask = j0 + G::kN > valid_min;
      float mx = kNegInf;
#pragma unroll
      for (int s = 0; s < G::kSub; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = sacc[s][i] * a.scale_log2;
          if (need_mask) {
            const int j = j0 + 32 * s + 8 * (i >> 2) + 4 * h + (i & 3);
            x = (j < bound) ? x : kNegInf;
          }
          sacc[s][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      m = m_new;
      // P^T operand per 16-key block kk: slots e = keys 16kk + 8(e/4) + 4h + e%4
      bf16x8 pop[G::kN / 16];
      float psum = 0.f, pexact = 0.f;
#pragma unroll
      for (int s = 0; s < G::kSub; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pe = exp2_fast(sacc[s][i] - m_use);
          const __bf16 pb = to_bf16(pe);
          pop[2 * s + (i >> 3)][i & 7] = pb;
          psum += bf16_to_f32(pb);
          pexact += pe;
        }
      lsum = alpha * lsum + psum;
      lexact = alpha * lexact + pexact;
#pragma unroll
      for (int nb = 0; nb < G::kNB; ++nb) oacc[nb] *= alpha;
      // ---- O^T += V^T P^T ----
      const int s16 = lane & 15;
      const int b16 = (lane >> 4) & 1;
#pragma unroll
      for (int kk = 0; kk < G::kN / 16; ++kk) {
        const __bf16 *v0 = vlds + (16 * kk + 4 * h + (s16 >> 2)) * G::kStride + 16 * b16 + 4 * (s16 & 3);
        const __bf16 *v1 = v0 + 8 * G::kStride;
#pragma unroll
        for (int nb = 0; nb < G::kNB; ++nb) {
          const bf16x4 lo = lds_read_tr16(v0 + 32 * nb);
          const bf16x4 hi = lds_read_tr16(v1 + 32 * nb);
          oacc[nb] = mfma32x32x16(concat(lo, hi), pop[kk], oacc[nb]);
        }
      }
    }

    if (more) {
      __bf16 *knext = lds + ((it + 1) & 1) * 2 * G::kTileElems;
      pf_store_tile<D>(knext, knext + G::kTileElems, tid, regs);
    }
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16; LSE2 = m + log2(l_exact) ----
  lsum += __shfl_xor(lsum, 32, 64);
  lexact += __shfl_xor(lexact, 32, 64);
  if (!row_valid) return;
  const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
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
    a.lse[(u.q_off + t) * a.num_q_heads + head] = (lexact > 0.f) ? muse + __log2f(lexact) : kNegInf;
  }
}

template <int D>
hipError_t launch_pf(const PrefillArgs &a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int gh = (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1);
  const int tq = kPfBlockRows / gh;
  const int64_t q_tiles = (a.max_seqlen_q + tq - 1) / tq;
  const int64_t blocks = q_tiles * a.batch * (a.num_q_heads / gh);
  hipLaunchKernelGGL(prefill_kernel<D>, dim3((unsigned)blocks), dim3(64 * kPfWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_pf<64>(a, stream);
    case 128: return launch_pf<128>(a, stream);
    case 256: return launch_pf<256>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace attn
