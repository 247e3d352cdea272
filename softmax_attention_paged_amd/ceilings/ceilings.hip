// Ceilings of the GPU measured with plain kernels, for the benchmark's
// secondary denominators (beside the published peaks): how fast a kernel can
// stream reads from HBM, how fast the matrix cores run a bf16 32x32x16 MFMA
// loop with no memory traffic (with fixed operands, and with operands that
// change every instruction), and how far the matrix and vector work of two
// waves on one SIMD overlap. Not part of the attention library: built into
// its own shared object, loaded by the benchmark only.
//
//   int ceil_stream_read(const void *src, size_t bytes, unsigned *sink,
//                        int blocks, hipStream_t stream);
//     reads every byte of src once (16-byte loads, four in flight per lane);
//     bytes must be a positive multiple of 16384 and src 16-byte aligned;
//     sink holds `blocks` words (written only on a value no input of zeros
//     and ones produces, so in practice never). Returns 0, or -1 on bad
//     arguments, or the HIP error code of the launch.
//   int ceil_mfma_bf16(float *sink, int iters, int blocks, hipStream_t stream);
//     each wave of `blocks` workgroups of four waves runs 4 * iters
//     independent-chain MFMAs (32768 flops each); sink holds blocks * 4
//     floats. Returns 0, -1 on bad arguments, or the HIP error code.
//   int ceil_mfma_bf16_varied(float *sink, int iters, int blocks, hipStream_t stream);
//     the same loop with every MFMA taking other operands: each lane holds
//     eight A and eight B operands of pseudo-random bf16 values (random
//     signs and mantissas, magnitudes in [0.25, 4)) and the four chains
//     cycle through them, so the matrix cores' inputs change every
//     instruction as they do in a real contraction (the loop above feeds the
//     same two operands to every MFMA). iters must be a positive multiple
//     of 8; otherwise the same arguments and returns.
//   int ceil_mfma_fma_overlap(float *sink, int kind, int mode, int n_mfma,
//                             int n_fma, int blocks, hipStream_t stream);
//     how far matrix and vector work of different waves overlap on one
//     SIMD: workgroups of eight waves, waves 0-3 (one per SIMD) run n_mfma
//     rounds of 32x32x16 (kind 0, four chains) or 16x16x32 (kind 1, eight
//     chains) bf16 MFMAs, the same number of flops either way, and waves
//     4-7 run n_fma rounds of eight independent FMA chains; mode 1 runs the
//     matrix waves only, 2 the vector waves only, 3 both. sink holds
//     blocks * 512 floats (written only on a value the loops never give).
//     Returns 0, -1 on bad arguments, or the HIP error code.
//   int ceil_lds_read(unsigned *sink, int kind, int iters, int blocks,
//                     hipStream_t stream);
//     LDS read bandwidth: workgroups of four waves fill 64 KB of LDS, then
//     each lane issues iters reads of 16 bytes (kind 0, ds_read_b128) or
//     two transposing 8-byte reads (kind 1, ds_read_b64_tr_b16), eight in
//     flight, the lanes of a wave on consecutive addresses (no bank
//     conflicts); every workgroup reads blocks * 256 * 16 * iters bytes in
//     all. iters must be a positive multiple of 8; sink holds blocks * 256
//     words (written only on a value the loop never gives).

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kGroup = 4 * kThreads;   // 16-byte chunks a workgroup reads per round

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ src, size_t groups,
                                                               unsigned *sink) {
  unsigned acc = 0;
  for (size_t g = blockIdx.x; g < groups; g += gridDim.x) {
    const u32x4 *p = src + g * kGroup + threadIdx.x;
    const u32x4 a = p[0], b = p[kThreads], c = p[2 * kThreads], d = p[3 * kThreads];
    acc ^= a.x ^ b.y ^ c.z ^ d.w ^ (a.w + b.x + c.y + d.z);
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__device__ __forceinline__ bool lane_is_zero() { return (threadIdx.x & 63) == 0; }

__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(float *sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.001f * (lane + e));
    b[e] = static_cast<__bf16>(0.002f * (lane - e));
  }
  f32x16 c0{}, c1{}, c2{}, c3{};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (lane == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = s;
}

// bf16 bits of a pseudo-random value: sign and mantissa from the hash,
// exponent so that |value| lies in [0.25, 4).
__device__ __forceinline__ unsigned short varied_bits(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  const unsigned exp = 125u + (x >> 7) % 4u;           // 2^-2 .. 2^1
  return static_cast<unsigned short>((x & 0x8000u) | (exp << 7) | (x & 0x7fu));
}

__global__ __launch_bounds__(kThreads) void mfma_varied_kernel(float *sink, int iters) {
  constexpr int kOps = 8;
  const unsigned seed = (blockIdx.x * kThreads + threadIdx.x) * 131u;
  bf16x8 a[kOps], b[kOps];
#pragma unroll
  for (int r = 0; r < kOps; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[r][e] = __builtin_bit_cast(__bf16, varied_bits(seed + 16u * r + e));
      b[r][e] = __builtin_bit_cast(__bf16, varied_bits(~(seed + 16u * r + e)));
    }
  f32x16 c0{}, c1{}, c2{}, c3{};
  for (int i = 0; i < iters; i += kOps) {
#pragma unroll
    for (int r = 0; r < kOps; ++r) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[r], b[(r + 1) % kOps], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 2) % kOps], b[(r + 3) % kOps], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 4) % kOps], b[(r + 5) % kOps], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(r + 6) % kOps], b[(r + 7) % kOps], c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (lane_is_zero()) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = s;
}

template <int KIND>
__global__ __launch_bounds__(512) void overlap_kernel(float *sink, int mode, int n_mfma, int n_fma) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool matrix_wave = wave < 4;
  if (matrix_wave ? !(mode & 1) : !(mode & 2)) return;
  float out = 0.f;
  if (matrix_wave) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = static_cast<__bf16>(0.001f * (lane + e));
      b[e] = static_cast<__bf16>(0.002f * (lane - e));
    }
    if constexpr (KIND == 0) {
      f32x16 c0{}, c1{}, c2{}, c3{};
      for (int i = 0; i < n_mfma; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) out += c0[i] + c1[i] + c2[i] + c3[i];
    } else {
      f32x4 c[8] = {};
      for (int i = 0; i < n_mfma; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) out += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    }
  } else {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.001f * (lane + j);
    const float m = 0.999f, add = 0.0001f * lane;
    for (int i = 0; i < n_fma; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __builtin_fmaf(x[j], m, add);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) out += x[j];
  }
  if (out == 12345.678f) sink[blockIdx.x * 512 + threadIdx.x] = out;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(256) void lds_read_kernel(unsigned *sink, int iters) {
  constexpr int kWords = 16384;                       // 64 KB
  __shared__ __attribute__((aligned(16))) unsigned buf[kWords];
  for (int i = threadIdx.x; i < kWords; i += 256) buf[i] = static_cast<unsigned>(i) * 2654435761u;
  __syncthreads();
  const unsigned base = threadIdx.x * 16u;            // 256 lanes x 16 bytes = 4 KB per round
  unsigned acc = 0;
  for (int i = 0; i < iters; i += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const unsigned off = (base + static_cast<unsigned>(i + u) * 4096u) & 0xffffu;
      const char *p = reinterpret_cast<const char *>(buf) + off;
      if constexpr (KIND == 0) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      } else {
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(reinterpret_cast<uintptr_t>(p)));
        const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(reinterpret_cast<uintptr_t>(p + 8)));
        acc ^= static_cast<unsigned>(a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w);
      }
    }
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

int ceil_stream_read(const void *src, size_t bytes, unsigned *sink, int blocks, hipStream_t stream) {
  if (!src || !sink || blocks < 1 || bytes == 0 || bytes % (16 * kGroup) ||
      reinterpret_cast<uintptr_t>(src) % 16)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4 *>(src), bytes / (16 * kGroup), sink);
  return static_cast<int>(hipGetLastError());
}

int ceil_mfma_bf16(float *sink, int iters, int blocks, hipStream_t stream) {
  if (!sink || iters < 1 || blocks < 1) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(kThreads), 0, stream, sink, iters);
  return static_cast<int>(hipGetLastError());
}

int ceil_mfma_bf16_varied(float *sink, int iters, int blocks, hipStream_t stream) {
  if (!sink || iters < 8 || iters % 8 || blocks < 1) return -1;
  hipLaunchKernelGGL(mfma_varied_kernel, dim3(blocks), dim3(kThreads), 0, stream, sink, iters);
  return static_cast<int>(hipGetLastError());
}

int ceil_mfma_fma_overlap(float *sink, int kind, int mode, int n_mfma, int n_fma, int blocks, hipStream_t stream) {
  if (!sink || kind < 0 || kind > 1 || mode < 1 || mode > 3 || n_mfma < 1 || n_fma < 1 || blocks < 1) return -1;
  if (kind == 0)
    hipLaunchKernelGGL(overlap_kernel<0>, dim3(blocks), dim3(512), 0, stream, sink, mode, n_mfma, n_fma);
  else
    hipLaunchKernelGGL(overlap_kernel<1>, dim3(blocks), dim3(512), 0, stream, sink, mode, n_mfma, n_fma);
  return static_cast<int>(hipGetLastError());
}

int ceil_lds_read(unsigned *sink, int kind, int iters, int blocks, hipStream_t stream) {
  if (!sink || kind < 0 || kind > 1 || iters < 8 || iters % 8 || blocks < 1) return -1;
  if (kind == 0)
    hipLaunchKernelGGL(lds_read_kernel<0>, dim3(blocks), dim3(256), 0, stream, sink, iters);
  else
    hipLaunchKernelGGL(lds_read_kernel<1>, dim3(blocks), dim3(256), 0, stream, sink, iters);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
