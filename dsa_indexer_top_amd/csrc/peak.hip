// Rate probes (dense MFMA loop, HBM copy and read, row gather) for measuring the path's
// kernels against peaks taken on the same GPU. Not part of the method.
#include <hip/hip_runtime.h>

#include "dsa_peak.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

// U 16-byte words per thread per round, loaded (nontemporal: read once)
// before any is used, so every wave keeps U loads in flight.
constexpr int kCopyU = 8;
constexpr int kReadU = 16;

__global__ __launch_bounds__(256) void copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (kCopyU - 1) * stride < n; i += kCopyU * stride) {
    u32x4 v[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read16(const u32x4* __restrict__ src, size_t n, uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0u;
  for (; i + (kReadU - 1) * stride < n; i += kReadU * stride) {
    u32x4 v[kReadU];
#pragma unroll
    for (int u = 0; u < kReadU; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadU; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += stride) {
    const u32x4 a = src[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
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

// Row gather: 256-byte rows table[idx[i]], each read by a group of 16 lanes
// (16 bytes per lane, four rows per wave instruction) and folded (xor) into
// out[block]. Each group keeps kGatherU rows in flight: their indices are
// loaded first, then the rows. An index outside [0, rows) reads row rows - 1.
constexpr int kGatherU = 16;

__global__ __launch_bounds__(256) void gather256(const u32x4* __restrict__ table, size_t rows,
                                                 const int* __restrict__ idx, size_t n, uint32_t* out) {
  const int c = threadIdx.x & 15;  // the lane's 16-byte chunk of a row
  const size_t groups = (size_t)gridDim.x * 16;
  size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  uint32_t x = 0u;
  for (; i + (kGatherU - 1) * groups < n; i += kGatherU * groups) {
    size_t r[kGatherU];
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) r[u] = min((size_t)(unsigned)idx[i + u * groups], rows - 1);
    u32x4 v[kGatherU];
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) v[u] = table[r[u] * 16 + c];
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += groups) {
    const u32x4 a = table[min((size_t)(unsigned)idx[i], rows - 1) * 16 + c];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
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
  hipLaunchKernelGGL(copy16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst,
                     bytes / 16);
  return launched();
}

extern "C" int dsa_peak_read(const void* src, size_t bytes, int blocks, uint32_t* out, void* stream) {
  if (!src || !out || bytes % 16 || blocks < 1 || (uintptr_t)src % 16) return 1;
  hipLaunchKernelGGL(read16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, bytes / 16, out);
  return launched();
}

extern "C" int dsa_peak_gather(const void* table, size_t rows, const int32_t* idx, size_t n, int blocks, uint32_t* out,
                               void* stream) {
  if (!table || !idx || !out || rows < 1 || n < 1 || blocks < 1 || (uintptr_t)table % 16 || (uintptr_t)idx % 4)
    return 1;
  hipLaunchKernelGGL(gather256, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)table, rows,
                     (const int*)idx, n, out);
  return launched();
}
