// Device-side building blocks for gfx950 (CDNA4): MFMA tiles, LDS transpose
// reads, exp2 and bf16 packing. Only the kernels of this library include it.
//
// Lane layouts (checked on gfx950 with an in-bounds probe before use):
//   v_mfma_f32_16x16x32_bf16, lane l, g = l / 16:
//     A (16 x 32): A[l % 16][8g + e], e = 0..7
//     B (32 x 16): B[8g + e][l % 16]
//     C (16 x 16): C[4g + i][l % 16], i = 0..3
//   v_mfma_f32_32x32x16_bf16, lane l, h = l / 32:
//     A: A[l % 32][8h + e]; B: B[8h + e][l % 32]
//     C: C[8(i / 4) + 4h + (i % 4)][l % 32], i = 0..15
//   ds_read_b64_tr_b16: within each 16-lane block, lane i receives element
//     (i % 4) of the 64-bit row addressed by lane (i / 4 + 4j) as its j-th
//     16-bit result, j = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even float -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }

// 16-byte global load of eight bf16 values.
__device__ __forceinline__ bf16x8 load_bf16x8(const void *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}

// 16-byte streaming load (non-temporal hint: data read once).
__device__ __forceinline__ bf16x8 load_bf16x8_stream(const void *p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}

__device__ __forceinline__ void store_bf16x8_lds(void *p, bf16x8 v) {
  *reinterpret_cast<u32x4 *>(p) = __builtin_bit_cast(u32x4, v);
}

// ds_read_b64_tr_b16 on an LDS address held in a generic pointer.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void *p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Direct HBM -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's bytes land at LDS byte address lds_base + 16 i; lds_base must be
// wave-uniform. Written as inline assembly so that the compiler, which
// cannot tell which LDS bytes the transfer writes, does not make later
// unrelated LDS reads wait for it: the caller waits (s_waitcnt vmcnt) and
// synchronises the workgroup before reading the destination.
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_base) : "memory");
}

// The same with a wave-uniform 64-bit base and a 32-bit per-lane byte
// offset (the saddr form: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void lds_dma16(const void *base, uint32_t lane_off, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(lane_off), "s"(base), "{m0}"(lds_base) : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Max / sum of a value over the two 32-lane halves of a wave, in every lane
// (v_permlane32_swap exchanges the halves).
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <class T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Key ranges of the GQA decode: the 32-key tiles a request's walk covers,
// [base, seq_len) with base the tile-aligned start of its window (0 without
// one), and at least one, so that a request without keys still belongs to a
// range whose waves write its empty rows. The split kernel and the merge
// both cut the batch with it.
__device__ __forceinline__ int gqa_request_tiles(int lk, int q_len, int window_left) {
  const int base = window_left >= 0 ? (max(0, lk - q_len - window_left) & ~31) : 0;
  return max(1, (lk - base + 31) >> 5);
}

// Tiles of every request, lane-strided (request lane + 64 k), and their sum
// over the batch (at most kKeyRangeMaxBatch requests); `below` sums only the
// requests before `b`.
struct BatchTiles {
  int n[kKeyRangeMaxBatch / 64];
  int total;
  int below;
};

__device__ __forceinline__ BatchTiles batch_tiles(const int32_t *seq_lens, int batch, int q_len, int window_left,
                                                  int b, int lane) {
  BatchTiles t;
  int sum = 0, below = 0;
#pragma unroll
  for (int k = 0; k < kKeyRangeMaxBatch / 64; ++k) {
    const int r = lane + 64 * k;
    t.n[k] = (r < batch) ? gqa_request_tiles(seq_lens[r], q_len, window_left) : 0;
    sum += t.n[k];
    below += (r < b) ? t.n[k] : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sum += __shfl_xor(sum, off, 64);
    below += __shfl_xor(below, off, 64);
  }
  t.total = sum;
  t.below = below;
  return t;
}

// Key range g of K over T tiles: [g T / K, (g + 1) T / K).
__device__ __forceinline__ int key_range_start(int g, int ranges, int total) {
  return (int)((int64_t)g * total / ranges);
}

// Exact e4m3 -> bf16 of 16 codes: one hardware convert per pair of codes, at
// scale 1 (every E4M3 value is a bf16 value; the OCP format on gfx950).
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 w, bf16x8 &lo, bf16x8 &hi) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const auto p01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], 1.0f, false);   // codes 0, 1
    const auto p23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], 1.0f, true);    // codes 2, 3
    bf16x8 &d = (q < 2) ? lo : hi;
    const int o = 4 * (q & 1);
    d[o + 0] = p01[0];
    d[o + 1] = p01[1];
    d[o + 2] = p23[0];
    d[o + 3] = p23[1];
  }
}

// Exact e4m3 -> bf16 of 8 codes.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  bf16x8 r;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const auto p01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], 1.0f, false);
    const auto p23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[q], 1.0f, true);
    r[4 * q + 0] = p01[0];
    r[4 * q + 1] = p01[1];
    r[4 * q + 2] = p23[0];
    r[4 * q + 3] = p23[1];
  }
  return r;
}

}  // namespace attn
