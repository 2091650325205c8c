// Paged KV cache maintenance: the new decode token's rows go to its request's
// last position, seq_lens[b] - 1, in a page pool (the step before the path).
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

__global__ __launch_bounds__(256) void paged_append_rows_kernel(const uint32_t* __restrict__ src, int words,
                                                                uint32_t* __restrict__ pool, PagedKV kv,
                                                                int max_seq_len) {
  const int b = blockIdx.x;
  const int len = decode_len(kv, b, 0, max_seq_len);
  if (len < 1) return;
  uint32_t* dst = pool + paged_row(kv, b, len - 1) * (size_t)words;
  const uint32_t* row = src + (size_t)b * words;
  for (int i = threadIdx.x; i < words; i += blockDim.x) dst[i] = row[i];
}

hipError_t launch_paged_append_rows(const void* src, int B, int row_bytes, void* pool, const PagedKV& kv,
                                    int max_seq_len, hipStream_t s) {
  hipLaunchKernelGGL(paged_append_rows_kernel, dim3(B), dim3(256), 0, s, (const uint32_t*)src, row_bytes / 4,
                     (uint32_t*)pool, kv, max_seq_len);
  return hipGetLastError();
}

}  // namespace dsa
