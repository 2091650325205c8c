// Cross-layer top-k overlap (IndexCache paper appendix, Figure 4: pairwise
// overlap of the layers' top-k index sets): for index tensors idx[l] [R, k],
//   inter[a][b] = sum_r |S_a(r) & S_b(r)|,  S_l(r) = valid entries of row r.
//
// One workgroup per (row r, layer a): row r of layer a is set as a bitmap of
// n_k bits in LDS, then row r of every layer b >= a is looked up in it, four
// layers per round so that their loads are in flight together. The four
// counts of a round are reduced over the workgroup and added to inter[a][b]
// and inter[b][a] with one 64-bit atomic each. The index rows are read from
// L2 (each is read by the n_layers workgroups of its row), so the kernel is
// bound by L2 reads: (n_layers + 1) * n_layers / 2 * k * 4 bytes per row.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kOverlapThreads = 256;
constexpr int kOverlapGroup = 4;  // layers b looked up per round

__global__ void overlap_zero_kernel(unsigned long long* __restrict__ a, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) a[i] = 0ull;
}

__global__ __launch_bounds__(kOverlapThreads) void topk_overlap_kernel(const int32_t* __restrict__ idx,
                                                                       int n_layers, int rows, int topk, int n_k,
                                                                       unsigned long long* __restrict__ inter) {
  extern __shared__ uint32_t bits[];  // ceil(n_k / 32) words
  __shared__ uint32_t part[kOverlapThreads / kWave][kOverlapGroup];
  const int r = blockIdx.x, a = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int words = (n_k + 31) >> 5;
  for (int i = threadIdx.x; i < words; i += kOverlapThreads) bits[i] = 0u;
  __syncthreads();
  const int32_t* ra = idx + ((size_t)a * rows + r) * topk;
  for (int j = threadIdx.x; j < topk; j += kOverlapThreads) {
    const int v = ra[j];
    if (v >= 0 && v < n_k) atomicOr(&bits[v >> 5], 1u << (v & 31));
  }
  __syncthreads();
  for (int b0 = a; b0 < n_layers; b0 += kOverlapGroup) {
    const int32_t* rb[kOverlapGroup];
#pragma unroll
    for (int q = 0; q < kOverlapGroup; ++q)
      rb[q] = idx + ((size_t)min(b0 + q, n_layers - 1) * rows + r) * topk;
    uint32_t c[kOverlapGroup] = {0u, 0u, 0u, 0u};
#pragma unroll 2
    for (int j = threadIdx.x; j < topk; j += kOverlapThreads) {
      int v[kOverlapGroup];
#pragma unroll
      for (int q = 0; q < kOverlapGroup; ++q) v[q] = rb[q][j];
#pragma unroll
      for (int q = 0; q < kOverlapGroup; ++q)
        c[q] += (v[q] >= 0 && v[q] < n_k) ? (bits[v[q] >> 5] >> (v[q] & 31)) & 1u : 0u;
    }
#pragma unroll
    for (int q = 0; q < kOverlapGroup; ++q) {
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) c[q] += __shfl_xor(c[q], d, 64);
      if (lane == 0) part[wave][q] = c[q];
    }
    __syncthreads();
    if (threadIdx.x < kOverlapGroup && b0 + (int)threadIdx.x < n_layers) {
      const int q = threadIdx.x, b = b0 + q;
      unsigned long long s = 0ull;
#pragma unroll
      for (int w = 0; w < kOverlapThreads / kWave; ++w) s += part[w][q];
      if (s) {
        atomicAdd(&inter[(size_t)a * n_layers + b], s);
        if (b != a) atomicAdd(&inter[(size_t)b * n_layers + a], s);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_topk_overlap(const int32_t* idx, int n_layers, int rows, int topk, int n_k, int64_t* inter,
                               hipStream_t s) {
  const int nn = n_layers * n_layers;
  hipLaunchKernelGGL(overlap_zero_kernel, dim3((nn + 255) / 256), dim3(256), 0, s, (unsigned long long*)inter, nn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)((n_k + 31) / 32) * 4;
  hipLaunchKernelGGL(topk_overlap_kernel, dim3(rows, n_layers), dim3(kOverlapThreads), lds, s, idx, n_layers, rows,
                     topk, n_k, (unsigned long long*)inter);
  return hipGetLastError();
}

}  // namespace dsa
