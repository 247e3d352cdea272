// FP8 (OCP E4M3) MLA-shaped ragged prefill over dense K/V, for gfx950:
// q, k 192 wide, v 128 wide, per-tensor dequantisation scales, bf16 output
// ("TokenSpeed-MLA": the prefill command's FP8 E4M3 inputs with q and k
// shapes [.., 192]; kernel capability summary: Q [sum q_lens, h_q, d_qk],
// K [sum kv_lens, h_k, d_qk], V [sum kv_lens, h_k, d_v], BF16 output,
// optional FP32 LSE).
//
// The structure follows the bf16 prefill kernel (four waves of 32 query rows,
// 64-key tiles, the scores of tile j+1 computed while tile j's softmax and
// P.V run, lazy re-base, bottom-right causal and sliding-window bounds).
// What changes with FP8:
//   - S^T = K Q^T runs on the FP8 matrix instruction v_mfma_f32_32x32x64
//     (E4M3 x E4M3, twice the bf16 rate): a lane holds 32 consecutive bytes
//     of one K row (A operand) and of one Q row (B operand), and the result
//     has the bf16 32x32 layout, so the softmax code is the bf16 one.
//   - K tiles move HBM -> LDS by direct loads, as codes (192-byte rows, the
//     16-byte chunks of row r XOR-swizzled by (r >> 2) & 3 so the 16 rows of
//     an operand read fall on distinct banks).
//   - V tiles pass through registers: each thread loads four 8-code pieces a
//     tile ahead, widens them exactly to bf16 and stores them into a bf16 LDS
//     tile laid out as the bf16 kernel's, so P.V is the same bf16 MFMA with
//     P rounded to bf16 (an E4M3 P would lose the row sums' precision).
//   - The q and k scales fold into the score scale, the v scale into the
//     final 1 / l.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_internal.h"
#include "device_common.h"
#include "prefill_unit.h"

namespace attn {
namespace {

constexpr int kF8W = 4;                                   // waves per workgroup
constexpr int kF8N = 64;                                  // keys per tile
constexpr int kF8Dqk = 192, kF8Dv = 128;
constexpr int kF8KB = kF8Dqk / 64;                        // QK k-steps of 64 codes
constexpr int kF8KRowB = kF8Dqk;                          // bytes of a K row (codes)
constexpr int kF8KChunks = kF8KRowB / 16;                 // 16-byte chunks per K row
constexpr int kF8KTileB = kF8N * kF8KRowB;                // bytes of a K tile
constexpr int kF8KLoads = kF8N * kF8KChunks / 64 / kF8W;  // direct loads per wave per K tile
constexpr int kF8VRowB = kF8Dv * 2;                       // bytes of a widened V row in LDS
constexpr int kF8VTileB = kF8N * kF8VRowB;                // bytes of a V tile in LDS
constexpr int kF8VPieces = kF8Dv / 8;                     // 8-code pieces per V row
constexpr int kF8VLoads = kF8N * kF8VPieces / (64 * kF8W);  // V pieces per thread per tile
constexpr int kF8NB = kF8Dv / 32;                         // PV 32-channel blocks
constexpr int kF8KK = kF8N / 16;                          // PV k-steps
static_assert(kF8N * kF8KChunks % (64 * kF8W) == 0, "whole K loads per wave");
static_assert(kF8N * kF8VPieces % (64 * kF8W) == 0, "whole V pieces per thread");

typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // format selectors 0, 0: both operands E4M3; zero scale operands give the
  // unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ int f8k_swz(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  i32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = static_cast<int>(lo[i]);
    r[4 + i] = static_cast<int>(hi[i]);
  }
  return r;
}

// S^T of the 64 keys of a K tile: two 32-key blocks x three 64-code k-steps.
__device__ __forceinline__ void f8_scores(const char *kbytes, const int (&koff)[kF8KB][2], const i32x8 (&qop)[kF8KB],
                                          f32x16 (&s)[2]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    s[sub] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < kF8KB; ++kb) {
      const char *p = kbytes + sub * 32 * kF8KRowB;
      const i32x8 a = cat8(*reinterpret_cast<const u32x4 *>(p + koff[kb][0]),
                           *reinterpret_cast<const u32x4 *>(p + koff[kb][1]));
      s[sub] = mfma_f8(a, qop[kb], s[sub]);
    }
  }
}

__device__ __forceinline__ float f8_max(const f32x16 (&s)[2]) {
  float mx = kNegInf;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sub][i]);
  return mx;
}

// Keys at or past `bound`, or before `begin` (this lane's row), get -inf.
__device__ __forceinline__ void f8_mask(f32x16 (&s)[2], int j0, int begin, int bound, int h) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + 32 * sub + 8 * (i >> 2) + 4 * h + (i & 3);
      s[sub][i] = (j < bound && j >= begin) ? s[sub][i] : kNegInf;
    }
}

__global__ __launch_bounds__(64 * kF8W, 2) void prefill_fp8_kernel(const PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kF8KTileB + 2 * kF8VTileB];   // K0 K1 V0 V1
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int r32 = lane & 31;

  PfUnit u;
  if (!pf_unit_xcd_heads<2>(a, kF8W, u)) return;   // two heads at a time per XCD: 2.25 -> 2.09 ms at 8K, 128 heads
  const int blocks_per_head = kF8W / u.gh;
  const int head = u.h0 + wave / blocks_per_head;
  const int t = u.q_end - u.tq + (wave % blocks_per_head) * 32 + r32;   // may be < 0 at the top
  const bool row_valid = t >= u.q_begin && t < u.q_end;
  int bound = a.causal ? min(u.lk, max(0, u.lk - u.lq + t + 1)) : u.lk;
  if (!row_valid) bound = 0;
  const bool windowed = a.window_left >= 0;
  const int begin = windowed ? max(0, u.lk - u.lq - a.window_left + t) : 0;
  const int jb = windowed ? max(0, u.lk - u.lq - a.window_left + u.q_begin) & ~(kF8N - 1) : 0;
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
  const int kv_end = a.causal ? min(u.lk, max(0, u.lk - u.lq + u.q_end)) : u.lk;
  const int nt = kv_end > jb ? (kv_end - jb + kF8N - 1) / kF8N : 0;       // tiles the workgroup loads
  const int ntw = wave_max > jb ? (wave_max - jb + kF8N - 1) / kF8N : 0;  // tiles this wave computes
  const int it0 = (windowed && begin_min != 0x7fffffff) ? (begin_min - jb) / kF8N : 0;

  // Q^T operand: 32 codes of this lane's row per k-step; a negative scale
  // flips the codes' sign bits (exact), so c > 0
  const float c = fabsf(a.scale_log2);
  const unsigned qsign = (a.scale_log2 < 0.f) ? 0x80808080u : 0u;
  i32x8 qop[kF8KB];
  {
    const uint8_t *qrow = static_cast<const uint8_t *>(a.q) + (u.q_off + t) * a.q_stride_tok +
                          (int64_t)head * a.q_stride_head;
#pragma unroll
    for (int kb = 0; kb < kF8KB; ++kb) {
      u32x4 lo = u32x4{0u, 0u, 0u, 0u}, hi = lo;
      if (row_valid) {
        lo = *reinterpret_cast<const u32x4 *>(qrow + 64 * kb + 32 * h);
        hi = *reinterpret_cast<const u32x4 *>(qrow + 64 * kb + 32 * h + 16);
      }
      const u32x4 sg = u32x4{qsign, qsign, qsign, qsign};
      qop[kb] = cat8(lo ^ sg, hi ^ sg);
    }
  }
  // K operand: chunks 4 kb + 2 h and + 1 of key r32 (+ 32 for the second block)
  int koff[kF8KB][2];
#pragma unroll
  for (int kb = 0; kb < kF8KB; ++kb)
#pragma unroll
    for (int p = 0; p < 2; ++p) koff[kb][p] = r32 * kF8KRowB + ((4 * kb + 2 * h + p) ^ f8k_swz(r32)) * 16;
  // V^T operand (transposing reads of the widened bf16 tile, as the bf16 kernel)
  int voff[2][kF8NB];
  {
    const int s16 = lane & 15;
    const int row0 = 4 * h + (s16 >> 2);
    const int cb = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
    const int f0 = pf_swz<kF8Dv>(row0), f1 = pf_swz<kF8Dv>(row0 + 8);
#pragma unroll
    for (int nb = 0; nb < kF8NB; ++nb) {
      voff[0][nb] = row0 * kF8VRowB + ((4 * nb + cb) ^ f0) * 16 + 8 * (s16 & 1);
      voff[1][nb] = (row0 + 8) * kF8VRowB + ((4 * nb + cb) ^ f1) * 16 + 8 * (s16 & 1);
    }
  }

  // K sources and this lane's direct-load offsets: load k of the wave fills
  // LDS chunk slot (k kW + wave) 64 + lane = row * 12 + physical chunk
  const uint8_t *ksrc = static_cast<const uint8_t *>(a.k) + u.kv_off * a.k_stride_tok + (int64_t)u.kvh * a.k_stride_head;
  const uint8_t *vsrc = static_cast<const uint8_t *>(a.v) + u.kv_off * a.v_stride_tok + (int64_t)u.kvh * a.v_stride_head;
  int krow[kF8KLoads], kchunk[kF8KLoads];
  uint32_t kdma_off[kF8KLoads];
#pragma unroll
  for (int k = 0; k < kF8KLoads; ++k) {
    const int slot = (k * kF8W + wave) * 64 + lane;
    krow[k] = slot / kF8KChunks;
    kchunk[k] = (slot % kF8KChunks) ^ f8k_swz(krow[k]);
    kdma_off[k] = static_cast<uint32_t>(krow[k] * a.k_stride_tok + kchunk[k] * 16);
  }
  auto kslot = [&](int par) { return lds + par * kF8KTileB; };
  auto vslot = [&](int par) { return lds + 2 * kF8KTileB + par * kF8VTileB; };
  auto issue_k = [&](int j0, char *dst) {
    const uint32_t base = lds_address(dst);
    if (j0 + kF8N <= u.lk) {
      const uint8_t *tile = ksrc + (int64_t)j0 * a.k_stride_tok;
#pragma unroll
      for (int k = 0; k < kF8KLoads; ++k) lds_dma16(tile, kdma_off[k], base + (k * kF8W + wave) * 1024);
    } else {
#pragma unroll
      for (int k = 0; k < kF8KLoads; ++k) {
        const int slot = (k * kF8W + wave) * 64 + lane;
        if (j0 + krow[k] < u.lk)   // lane L of the load lands at the load's base + 16 L
          lds_dma16(ksrc + (int64_t)(j0 + krow[k]) * a.k_stride_tok + kchunk[k] * 16, base + (k * kF8W + wave) * 1024);
        else
          *reinterpret_cast<u32x4 *>(dst + slot * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // V: thread piece q = k * 256 + tid is row q / 16, codes 8 (q % 16) .. + 7,
  // widened to the row's bf16 chunk q % 16: the 16 lanes of a quarter-wave
  // write one whole 256-byte row, every bank once. Rows past the request are
  // zero (P is 0 there, and 0 * NaN would not be).
  u32x2 vstage[kF8VLoads];
  auto load_v = [&](int j0) {
#pragma unroll
    for (int k = 0; k < kF8VLoads; ++k) {
      const int q = k * 64 * kF8W + tid;
      const int row = q / kF8VPieces, pc = q % kF8VPieces;
      vstage[k] = (j0 + row < u.lk)
                      ? *reinterpret_cast<const u32x2 *>(vsrc + (int64_t)(j0 + row) * a.v_stride_tok + pc * 8)
                      : u32x2{0u, 0u};
    }
  };
  auto store_v = [&](char *dst) {
#pragma unroll
    for (int k = 0; k < kF8VLoads; ++k) {
      const int q = k * 64 * kF8W + tid;
      const int row = q / kF8VPieces, pc = q % kF8VPieces;
      store_bf16x8_lds(dst + row * kF8VRowB + (pc ^ pf_swz<kF8Dv>(row)) * 16, fp8x8_to_bf16(vstage[k]));
    }
  };

  if (nt > 0) {
    issue_k(jb, kslot(0));
    load_v(jb);
    if (nt > 1) issue_k(jb + kF8N, kslot(1));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_v(vslot(0));
    if (nt > 1) load_v(jb + kF8N);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  f32x16 s[2];
  float mx = kNegInf;
  if (ntw > 0) {
    f8_scores(kslot(0), koff, qop, s);
    mx = f8_max(s);
  }
  float m = kNegInf, lsum = 0.f;
  f32x16 oacc[kF8NB];
#pragma unroll
  for (int nb = 0; nb < kF8NB; ++nb) oacc[nb] = f32x16{};

  // Unrolled by two so each half knows its LDS slots at compile time (see the
  // bf16 kernel); the per-lane offsets are made opaque once per tile.
  auto tile_step = [&](int it, auto par_c) {
    constexpr int par = decltype(par_c)::value;
#pragma unroll
    for (int kb = 0; kb < kF8KB; ++kb) asm volatile("" : "+v"(koff[kb][0]), "+v"(koff[kb][1]));
#pragma unroll
    for (int nb = 0; nb < kF8NB; ++nb) asm volatile("" : "+v"(voff[0][nb]), "+v"(voff[1][nb]));
    // K(it+1) has landed and V(it) is stored for every wave; every wave is
    // done with K(it) and V(it-1), whose slots take K(it+2) and V(it+1); the
    // staged codes of V(it+1) have landed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int j0 = jb + it * kF8N;
    if (it + 2 < nt) issue_k(j0 + 2 * kF8N, kslot(par));
    if (it + 1 < nt) store_v(vslot(par ^ 1));
    if (it + 2 < nt) load_v(j0 + 2 * kF8N);
    // (a wave whose window starts in tile it0 skips the tiles before it0 - 1,
    // as in the bf16 kernel)
    if ((unsigned)(it + 1 - it0) < (unsigned)(ntw + 1 - it0)) {
      if (j0 + kF8N > valid_min || j0 < begin_max) {
        f8_mask(s, j0, begin, bound, h);
        mx = f8_max(s);
      }
      const float mt = half_max(mx) * c;
      const float m_new = (mt > m + kRebase) ? mt : m;
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      m = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int nb = 0; nb < kF8NB; ++nb) oacc[nb] *= alpha;
      }
      // S(it+1) on the FP8 matrix cores beside P(it) on the vector units
      f32x16 sn[2];
      f8_scores(kslot(par ^ 1), koff, qop, sn);
      bf16x8 pop[kF8KK];
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pe = exp2_fast(__builtin_fmaf(s[sub][i], c, -m_use));
          pop[2 * sub + (i >> 3)][i & 7] = to_bf16(pe);
          ps[i & 1] += pe;
        }
      const char *vbytes = vslot(par);
#pragma unroll
      for (int kk = 0; kk < kF8KK; ++kk)
#pragma unroll
        for (int nb = 0; nb < kF8NB; ++nb) {
          const bf16x4 lo = lds_read_tr16(vbytes + voff[0][nb] + kk * 16 * kF8VRowB);
          const bf16x4 hi = lds_read_tr16(vbytes + voff[1][nb] + kk * 16 * kF8VRowB);
          oacc[nb] = mfma32x32x16(concat(lo, hi), pop[kk], oacc[nb]);
        }
      lsum = alpha * lsum + (ps[0] + ps[1]);
      s[0] = sn[0];
      s[1] = sn[1];
      mx = f8_max(s);
    }
  };
  for (int it = 0; it < nt; it += 2) {
    tile_step(it, std::integral_constant<int, 0>{});
    if (it + 1 < nt) tile_step(it + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O * v_scale / l -> bf16; LSE2 = m + log2(l) ----
  const float l = half_sum(lsum);
  if (!row_valid) return;
  const float inv = (l > 0.f) ? a.v_scale / l : 0.f;
  __bf16 *orow = static_cast<__bf16 *>(a.o) + (u.q_off + t) * a.o_stride_tok + (int64_t)head * a.o_stride_head;
#pragma unroll
  for (int nb = 0; nb < kF8NB; ++nb)
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

}  // namespace

hipError_t launch_prefill_fp8(const PrefillArgs &a, hipStream_t stream) {
  if (a.block_table || a.head_dim != kF8Dqk) return hipErrorNotSupported;
  const int gh = pf_heads_per_wg(a.num_q_heads / a.num_kv_heads);
  const int tq = 32 * kF8W / gh;
  const int64_t q_tiles = (a.max_seqlen_q + tq - 1) / tq;
  const int64_t blocks = q_tiles * a.batch * (a.num_q_heads / gh);
  hipLaunchKernelGGL(prefill_fp8_kernel, dim3((unsigned)blocks), dim3(64 * kF8W), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
