// The step before attention reads its inputs, for gfx950: the K/V cache
// append ("Writing Page Attention with PyPTO", sections 4.2-4.3 and 9.2) and
// the MLA K/V pack + FP8 quantise ("TokenSpeed-MLA", kernel capability
// summary). Both move bytes and do almost no arithmetic, so both are laid
// out for HBM: every lane moves one 16-byte chunk of 8 bf16 values (8 bytes
// out when quantised) at a time, with four chunks' loads issued before their
// stores so enough bytes are in flight to cover HBM latency; the lanes of a
// wave cover consecutive chunks of a row, and one workgroup owns one token
// so its rows are read and written as whole contiguous runs.
//
// E4M3 quantisation: y = x / scale as the correctly rounded binary32 quotient
// (see div_rn), clamped to
// +-448 (E4M3 has no infinity; the clamp keeps NaN, whose comparisons are
// false), then converted by the hardware's round-to-nearest-even fp32 ->
// OCP E4M3 conversion.

#include <hip/hip_runtime.h>

#include "attn_internal.h"
#include "device_common.h"

namespace attn {
namespace {

constexpr int kPrologueThreads = 256;
constexpr int kBatch = 4;              // 16-byte chunks each lane loads before it stores
constexpr float kE4m3Max = 448.0f;
constexpr int kMaxRopeChunks = 4096 / 8;   // d_nope + d_rope <= 4096

// x / scale rounded once to binary32, from inv = RN(1 / scale): q0 = x * inv
// is within one ulp of the quotient, and one fma correction with the exact
// remainder x - q0 * scale gives the correctly rounded quotient (Markstein's
// theorem on division with a correctly rounded reciprocal; valid while no
// step overflows or underflows). Quotients beyond 2^20 saturate whatever
// their last bit, so they skip the correction (whose remainder could
// overflow); copysign keeps the sign of a zero quotient. The result is then
// clamped to +-448 (E4M3 has no infinity).
__device__ __forceinline__ float div_sat(float x, float scale, float inv) {
  const float q0 = x * inv;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, scale, x), inv, q0);
  const float y = __builtin_copysignf(__builtin_fabsf(q0) < 0x1p20f ? q : q0, q0);
  return __builtin_amdgcn_fmed3f(y, -kE4m3Max, kE4m3Max);
}

// 8 bf16 values / scale -> 8 E4M3 codes (byte e holds value e).
__device__ __forceinline__ u32x2 quantize8(bf16x8 x, float scale, float inv) {
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = div_sat(static_cast<float>(x[e]), scale, inv);
  u32x2 r;
  int w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], w1, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  r[0] = static_cast<unsigned>(w0);
  r[1] = static_cast<unsigned>(w1);
  return r;
}

// One workgroup per new token: chunk c of the token's K heads, then of its
// V heads. The destination row is the clamped slot plus the layer base.
template <bool FP8>
__global__ __launch_bounds__(kPrologueThreads) void cache_append_kernel(const CacheAppendArgs a) {
  const int tok = blockIdx.x;
  const int64_t slot = a.slot_mapping[tok];
  const int64_t row = a.layer_base_rows + (slot > 0 ? slot : 0);
  if (row >= a.num_cache_rows) return;                 // uniform
  const int64_t page = row >> a.page_shift;
  const int64_t in_page = row & ((int64_t(1) << a.page_shift) - 1);
  const int kc = a.head_dim_k / 8, vc = a.head_dim_v / 8;
  const int k_chunks = a.num_kv_heads * kc;
  const int total = k_chunks + (a.v_new ? a.num_kv_heads * vc : 0);
  const float k_inv = 1.0f / a.k_scale, v_inv = 1.0f / a.v_scale;   // IEEE quotients
  for (int base = 0; base < total; base += kBatch * kPrologueThreads) {
    bf16x8 x[kBatch];
    int64_t dst_off[kBatch];
    bool is_k[kBatch], live[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * kPrologueThreads + threadIdx.x;
      live[u] = i < total;
      if (!live[u]) continue;
      is_k[u] = i < k_chunks;
      const int j = is_k[u] ? i : i - k_chunks;
      const int per = is_k[u] ? kc : vc;
      const int head = j / per, c = j % per;
      const __bf16 *src = static_cast<const __bf16 *>(is_k[u] ? a.k_new : a.v_new) +
                          tok * (is_k[u] ? a.k_new_stride_tok : a.v_new_stride_tok) +
                          head * (is_k[u] ? a.k_new_stride_head : a.v_new_stride_head) + c * 8;
      dst_off[u] = page * (is_k[u] ? a.k_stride_page : a.v_stride_page) +
                   in_page * (is_k[u] ? a.k_stride_tok : a.v_stride_tok) +
                   head * (is_k[u] ? a.k_stride_head : a.v_stride_head) + c * 8;
      x[u] = load_bf16x8(src);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (!live[u]) continue;
      if constexpr (FP8) {
        uint8_t *dst = static_cast<uint8_t *>(is_k[u] ? a.k_cache : a.v_cache) + dst_off[u];
        *reinterpret_cast<u32x2 *>(dst) = is_k[u] ? quantize8(x[u], a.k_scale, k_inv) : quantize8(x[u], a.v_scale, v_inv);
      } else {
        __bf16 *dst = static_cast<__bf16 *>(is_k[u] ? a.k_cache : a.v_cache) + dst_off[u];
        *reinterpret_cast<u32x4 *>(dst) = __builtin_bit_cast(u32x4, x[u]);
      }
    }
  }
}

// Quantise one region of a token's rows: `heads` rows of `chunks` 16-byte
// chunks, row h read at src + h * src_stride and written at dst + h *
// dst_stride (element strides, both
// below 2^24 so 24-bit multiplies address them). kBatch chunks per lane per
// round: all loads first, then the stores, so each lane keeps kBatch 16-byte
// reads in flight; a lane's (row, chunk) position advances by a fixed step.
__device__ __forceinline__ void pack_region(const __bf16 *src, int src_stride, uint8_t *dst, int dst_stride,
                                            int heads, int chunks, float scale, float inv) {
  const int total = heads * chunks;
  const int step_h = kPrologueThreads / chunks, step_c = kPrologueThreads % chunks;
  int h = threadIdx.x / chunks, c = threadIdx.x % chunks;
  for (int base = 0; base < total; base += kBatch * kPrologueThreads) {
    bf16x8 x[kBatch];
    uint32_t off[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool live = base + u * kPrologueThreads + static_cast<int>(threadIdx.x) < total;
      off[u] = live ? __umul24(h, dst_stride) + c * 8 : ~0u;
      if (live) x[u] = load_bf16x8(src + __umul24(h, src_stride) + c * 8);
      h += step_h;
      c += step_c;
      if (c >= chunks) {
        c -= chunks;
        ++h;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (off[u] != ~0u) *reinterpret_cast<u32x2 *>(dst + off[u]) = quantize8(x[u], scale, inv);
  }
}

// Quantise a token's K rows whole: row h has `chunks` 8-byte output chunks,
// the first `src_chunks` from the 16-byte chunks of src + h * src_stride,
// the rest copied from `rope_codes` (the shared rope row, quantised once).
// Each wave's stores cover consecutive chunks of consecutive rows, so a row
// is written in one pass rather than as a head and a tail at different times.
__device__ __forceinline__ void pack_k_rows(const __bf16 *src, int src_stride, uint8_t *dst, int dst_stride,
                                            int heads, int chunks, int src_chunks, const u32x2 *rope_codes,
                                            float scale, float inv) {
  const int total = heads * chunks;
  const int step_h = kPrologueThreads / chunks, step_c = kPrologueThreads % chunks;
  int h = threadIdx.x / chunks, c = threadIdx.x % chunks;
  for (int base = 0; base < total; base += kBatch * kPrologueThreads) {
    bf16x8 x[kBatch];
    uint32_t off[kBatch];
    int rc[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool live = base + u * kPrologueThreads + static_cast<int>(threadIdx.x) < total;
      off[u] = live ? __umul24(h, dst_stride) + c * 8 : ~0u;
      rc[u] = c - src_chunks;
      if (live && rc[u] < 0) x[u] = load_bf16x8(src + __umul24(h, src_stride) + c * 8);
      h += step_h;
      c += step_c;
      if (c >= chunks) {
        c -= chunks;
        ++h;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (off[u] != ~0u)
        *reinterpret_cast<u32x2 *>(dst + off[u]) = rc[u] < 0 ? quantize8(x[u], scale, inv) : rope_codes[rc[u]];
  }
}

// One workgroup per token: the token's rope row is quantised once into LDS
// (its codes are the same for every head), then every K row is written
// whole (d_nope bytes from k_nope, d_rope bytes of rope codes), then the V
// rows.
__global__ __launch_bounds__(kPrologueThreads) void mla_kv_pack_kernel(const MlaPackArgs a) {
  __shared__ u32x2 rope_codes[kMaxRopeChunks];
  const int64_t tok = blockIdx.x;
  const float k_inv = 1.0f / a.k_scale, v_inv = 1.0f / a.v_scale;   // IEEE quotients
  const int nch = a.d_nope / 8, rch = a.d_rope / 8;
  if (rch > 0) {
    const __bf16 *rope = static_cast<const __bf16 *>(a.k_rope) + tok * a.k_rope_stride_tok;
    for (int i = threadIdx.x; i < rch; i += kPrologueThreads)
      rope_codes[i] = quantize8(load_bf16x8(rope + i * 8), a.k_scale, k_inv);
  }
  __syncthreads();
  pack_k_rows(static_cast<const __bf16 *>(a.k_nope) + tok * a.k_nope_stride_tok, static_cast<int>(a.k_nope_stride_head),
              static_cast<uint8_t *>(a.k_out) + tok * a.k_out_stride_tok, static_cast<int>(a.k_out_stride_head),
              a.num_heads, nch + rch, nch, rope_codes, a.k_scale, k_inv);
  pack_region(static_cast<const __bf16 *>(a.v) + tok * a.v_stride_tok, static_cast<int>(a.v_stride_head),
              static_cast<uint8_t *>(a.v_out) + tok * a.v_out_stride_tok, static_cast<int>(a.v_out_stride_head),
              a.num_heads, a.d_v / 8, a.v_scale, v_inv);
}

}  // namespace

hipError_t launch_cache_append(const CacheAppendArgs &a, hipStream_t stream) {
  if (a.fp8)
    hipLaunchKernelGGL(cache_append_kernel<true>, dim3(a.num_tokens), dim3(kPrologueThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(cache_append_kernel<false>, dim3(a.num_tokens), dim3(kPrologueThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mla_kv_pack(const MlaPackArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(mla_kv_pack_kernel, dim3(a.num_tokens), dim3(kPrologueThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn
