// Rate probes (dense MFMA loop, HBM copy and read) for measuring the path's
// kernels against peaks taken on the same GPU. Not part of the method.
#include <hip/hip_runtime.h>

#include "dsa_peak.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Four independent accumulator chains per wave keep the matrix pipe fed
// across each MFMA's latency; two workgroups of four waves per CU put two
// waves on every SIMD.
template <bool FP8>
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* out) {
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  const int t = threadIdx.x;
  if constexpr (FP8) {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38303830 + ((t + i) & 7);  // e4m3 codes near 1.0
      b[i] = 0x30383038 + ((t * 3 + i) & 7);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(1.0f + 0.001f * ((t + i) & 7));
      b[i] = (__bf16)(0.5f - 0.001f * ((t * 3 + i) & 7));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * 256 + t] = s;
}

// Four 16-byte words per thread per round, so every wave has four loads in
// flight before its stores.
__global__ __launch_bounds__(256) void copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read16(const uint4* __restrict__ src, size_t n, uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0u;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int d = 128; d >= 1; d >>= 1) {
    if ((int)threadIdx.x < d) red[threadIdx.x] ^= red[threadIdx.x + d];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : 2; }

}  // namespace

extern "C" int dsa_peak_mfma(int dtype, int blocks, int iters, float* out, double* flop, void* stream) {
  if ((dtype != 0 && dtype != 1) || blocks < 1 || iters < 1 || !out) return 1;
  hipStream_t s = (hipStream_t)stream;
  const double per = dtype == 1 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
  if (flop) *flop = per * 4.0 * iters * 4.0 * blocks;  // 4 chains x 4 waves per block
  if (dtype == 1)
    hipLaunchKernelGGL(mfma_loop<true>, dim3(blocks), dim3(256), 0, s, iters, out);
  else
    hipLaunchKernelGGL(mfma_loop<false>, dim3(blocks), dim3(256), 0, s, iters, out);
  return launched();
}

extern "C" int dsa_peak_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes % 16 || blocks < 1 || ((uintptr_t)src | (uintptr_t)dst) % 16) return 1;
  hipLaunchKernelGGL(copy16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, (uint4*)dst,
                     bytes / 16);
  return launched();
}

extern "C" int dsa_peak_read(const void* src, size_t bytes, int blocks, uint32_t* out, void* stream) {
  if (!src || !out || bytes % 16 || blocks < 1 || (uintptr_t)src % 16) return 1;
  hipLaunchKernelGGL(read16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, bytes / 16, out);
  return launched();
}
