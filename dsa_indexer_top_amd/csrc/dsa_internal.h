// Internal interface between the host API (dsa_api.cpp) and the kernel
// launchers (*.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Candidate-list capacity per query row, 4k (at least k + 512), in both
// paths. Prefill (streaming filter): room for the kept superset of the top-k
// plus the 256 appends a nearly full list may still receive before its shrink;
// a shrink costs about C / (C - k) list passes per accepted key. Decode (one
// threshold pass): every key whose 12-bit histogram bin reaches the k-th
// key's bin, i.e. k plus most of one bin; a larger list sends the request to
// the exact full-row select.
inline int cand_capacity(int topk, bool decode) {
  (void)decode;
  int c = topk * 4;
  if (c < topk + 512) c = topk + 512;
  return (c + 63) / 64 * 64;
}

// Decode path: bins of the first-level histogram of the 32-bit score keys.
constexpr int kDecodeHistBits = 12;
constexpr int kDecodeHistBins = 1 << kDecodeHistBits;
constexpr int kDecodeCoarseBins = 64;  // sums of 64 consecutive bins, stored after them
// Each request's row: the fine bins, the coarse bins, then its candidate
// counter alone in the last 256 bytes (the requests' counters sit a row
// apart, so the collect blocks' atomics on them do not queue on one line).
constexpr int kDecodeCntOffset = kDecodeHistBins + kDecodeCoarseBins;
constexpr int kDecodeHistStride = kDecodeCntOffset + 64;
// A request's histogram is kept in kDecodeHistCopies copies (score block j
// adds to copy j mod kDecodeHistCopies), so the blocks' atomics on the few
// bins that hold most keys queue on eight addresses instead of one; readers
// sum the copies. The request's counter is the one in copy 0.
constexpr int kDecodeHistCopies = 8;
constexpr int kDecodeHistRow = kDecodeHistCopies * kDecodeHistStride;
// Row stride of the decode score keys: n_k rounded up to 64 keys (256 B), so
// every row starts aligned and 16-key vector reads stay inside it.
__host__ __device__ inline size_t decode_key_stride(int n_k) { return ((size_t)n_k + 63) / 64 * 64; }
constexpr int kDecodeWaveKeys = 32;          // keys per wave step of the score kernel
constexpr int kDecodeBlockKeys = 4 * kDecodeWaveKeys;
constexpr int kDecodeCollectKeys = 4096;     // keys per block of the collect kernel
constexpr int kDecodeTargetBlocks = 256;     // score blocks per decode call (one per CU)

// Paged, ragged decode: token s of request b is row
// block_table[b * max_pages + s / page_size] * page_size + s % page_size of the
// pools; request b has seq_lens[b] tokens. block_table == nullptr: flat layout.
struct PagedKV {
  const int32_t* seq_lens;
  const int32_t* block_table;
  int page_size, max_pages, num_pages;
};

// Decode context length of request b (clamped to [0, n_k]), or the flat one.
__device__ __forceinline__ int decode_len(const PagedKV& kv, int b, int pos_offset, int n_k) {
  if (kv.seq_lens) {
    const int s = kv.seq_lens[b];
    return s < 0 ? 0 : (s > n_k ? n_k : s);
  }
  return min(pos_offset + 1, n_k);
}

// Pool row of token s of request b (page id clamped into the pool).
__device__ __forceinline__ size_t paged_row(const PagedKV& kv, int b, int s) {
  int page = kv.block_table[(size_t)b * kv.max_pages + s / kv.page_size];
  page = page < 0 ? 0 : (page >= kv.num_pages ? kv.num_pages - 1 : page);
  return (size_t)page * kv.page_size + s % kv.page_size;
}

struct IndexerParams {
  int B, n_q, n_k, pos_offset, H, D, topk, fp8;
  const void* q;
  const void* k;
  const float* w;
  const float* q_scale;
  const float* k_scale;
  int32_t* out_idx;
  float* out_scores;
  float* dump;
  // workspace views
  uint32_t* cand_key;   // [rows, C]
  int32_t* cand_idx;    // [rows, C]
  int32_t* cand_cnt;    // [rows], row r at cand_cnt[r * cnt_stride]
  int cnt_stride;       // 1 (prefill) or kDecodeHistRow (decode: inside the histogram rows)
  int C;
  uint32_t* dec_keys;   // decode: [B, dec_stride] score keys
  uint32_t* dec_hist;   // decode: [B, kDecodeHistCopies, kDecodeHistStride] (fine bins, coarse bins, counter)
  int32_t* dec_work;    // decode: [B + kDecodeTargetBlocks, 3] (request, k0, k1) per score
                        // block, planned on the device when lengths are ragged (kv.seq_lens)
  PagedKV kv;           // decode only: paged pools (kv.block_table) or flat
  void* const* ev;      // optional phase events (3): before scores, after scores, after select
  int skip_prepare;     // decode: histograms and counters already zero and the ragged
                        // plan already built for this kv (a later F layer of a stack)
};

// Records phase event i (if any) on the stream.
inline hipError_t record_phase(void* const* ev, int i, hipStream_t s) {
  return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess;
}

struct AttnParams {
  int B, n_q, n_k, pos_offset, H, D, topk;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  void* out;
  float* lse;
  int nsplit;           // waves that share one row's idx list (split-K), attn_nsplit
  float* part;          // [rows, attn_nparts(nsplit), H, kAttnPartStride]: O[D], max, sum, pad
  PagedKV kv;           // decode only: paged pools (kv.block_table) or flat
  void* const* ev;      // optional phase events (2): before, after
};

// floats per (query, split, head) partial of split attention: O[D], max, sum,
// padded so every partial starts 16-byte aligned
template <int D>
constexpr int kAttnPartStride = D + 4;
inline int attn_part_stride(int D) { return D + 4; }

size_t indexer_workspace_bytes(int B, int n_q, int n_k, int topk);
size_t indexer_decode_plan_offset(int B, int n_k, int topk);
size_t attn_workspace_bytes(int B, int n_q, int n_k, int H, int D, int topk);
int attn_nsplit(int B, int n_q, int topk);
// Waves per workgroup that merge their splits in LDS, and the partials per
// row the merge kernel reads for nsplit splits: none for one split (the wave
// writes the output), one per wave below kAttnGroupSplits splits, one per
// workgroup from there on: at exactly kAttnGroupSplits splits one workgroup
// of that many waves writes the output directly (1 partial); from twice that
// on, workgroups of 4 waves each write one partial (at most 16 per row, at
// 64 splits), which starts and merges a decode call's waves in smaller groups.
constexpr int kAttnGroupSplits = 8;
constexpr int kAttnMaxParts = 16;
__host__ __device__ inline int attn_group_waves(int nsplit) { return nsplit > kAttnGroupSplits ? 4 : kAttnGroupSplits; }
__host__ __device__ inline int attn_nparts(int nsplit) {
  return nsplit >= kAttnGroupSplits ? nsplit / attn_group_waves(nsplit) : nsplit;
}

// Carves the workspace into the views above.
void indexer_bind_workspace(IndexerParams& p, void* ws);

hipError_t launch_indexer_prefill(const IndexerParams& p, hipStream_t s);
hipError_t launch_indexer_decode(const IndexerParams& p, hipStream_t s);
hipError_t launch_sparse_attn(const AttnParams& p, hipStream_t s);
hipError_t launch_paged_append_rows(const void* src, int B, int row_bytes, void* pool, const PagedKV& kv,
                                    int max_seq_len, hipStream_t s);
hipError_t launch_topk_overlap(const int32_t* idx, int n_layers, int rows, int topk, int n_k, int64_t* inter,
                               hipStream_t s);
hipError_t launch_quantize_fp8_rows(const void* x, int64_t rows, int cols, void* out, float* scale, hipStream_t s);

}  // namespace dsa
