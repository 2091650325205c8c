// Exact per-row top-k finalisation and the decode-path selection kernels.
//
// Order used everywhere: the 64-bit composite key (score_key(score) << 32) |
// ~index, larger = better, i.e. higher score first and, for equal scores,
// lower index first. Composite keys are unique, so "the first k in composite
// order" is exactly the top-k with the library's tie rule.
#include "dsa_device.h"
#include "dsa_internal.h"

#include <type_traits>

namespace dsa {

constexpr int kFinNT = 256;
constexpr int kFinMax = 4096;  // largest candidate list sorted in LDS

__device__ __forceinline__ uint64_t composite(uint32_t u, int32_t idx) {
  return ((uint64_t)u << 32) | (uint64_t)(~(uint32_t)idx);
}

// Descending bitonic sort of s[0..n) (n a power of two) by the whole workgroup.
__device__ void block_bitonic_desc(uint64_t* s, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) != 0;  // this pair's segment is ascending
        const uint64_t a = s[lo], c = s[hi];
        if (up ? (a > c) : (a < c)) {
          s[lo] = c;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Block-wide exclusive prefix sum of one value per thread (blockDim.x <= 1024).
__device__ int block_excl_scan(int v, int* scratch /* >= 17 ints */, int* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t incl = wave_incl_scan((uint32_t)v);
  if (lane == 63) scratch[wave] = (int)incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < nw; ++w) {
      const int x = scratch[w];
      scratch[w] = acc;
      acc += x;
    }
    scratch[16] = acc;
  }
  __syncthreads();
  const int r = scratch[wave] + (int)incl - v;
  *total = scratch[16];
  __syncthreads();
  return r;
}

// The k-th largest of keys[0..n) (1 <= k <= n), by 4 radix steps of 8 bits
// over a 256-bin LDS histogram: *theta = that key, *need = how many keys equal
// to theta belong to the k largest when ties go to the lowest index.
// keys may live in LDS or global memory. Called by the whole workgroup.
__device__ void block_kth_key(const uint32_t* keys, int n, int k, uint32_t* hist, uint32_t* theta,
                              int* need) {
  __shared__ int sh_digit, sh_above;
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t u = keys[i];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      const int hb = 255 - 4 * lane;  // lane order = descending digit order
      const uint32_t c0 = hist[hb], c1 = hist[hb - 1], c2 = hist[hb - 2], c3 = hist[hb - 3];
      const uint32_t loc = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_incl_scan(loc);
      const uint32_t rem = (uint32_t)remaining;
      const uint64_t m = ballot(incl >= rem);
      const int L = uniform_i(m ? __builtin_ctzll(m) : 63);
      const uint32_t cum = incl - loc;
      int digit;
      uint32_t above;
      if (cum + c0 >= rem) {
        digit = hb; above = cum;
      } else if (cum + c0 + c1 >= rem) {
        digit = hb - 1; above = cum + c0;
      } else if (cum + c0 + c1 + c2 >= rem) {
        digit = hb - 2; above = cum + c0 + c1;
      } else {
        digit = hb - 3; above = cum + c0 + c1 + c2;
      }
      if (lane == L) {
        sh_digit = digit;
        sh_above = (int)above;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh_digit << shift;
    pmask |= 0xFFu << shift;
    remaining -= sh_above;
    __syncthreads();
  }
  *theta = prefix;
  *need = remaining;
}

// Writes, in list order, the composite keys of the entries of keys[0..n) that
// are > theta plus the first `need` equal to theta, to s[0..). idx[i] is the
// token index of entry i (NULL: the entry's position). Each thread owns one
// contiguous segment, so two block-wide scans place every entry.
__device__ void block_ordered_collect(const uint32_t* keys, const int32_t* __restrict__ idx, int n,
                                      uint32_t theta, int need, uint64_t* s, int* scratch) {
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int i0 = min((int)threadIdx.x * per, n), i1 = min(i0 + per, n);
  int ties = 0;
  for (int i = i0; i < i1; ++i) ties += keys[i] == theta;
  int tie_total;
  int tie_rank = block_excl_scan(ties, scratch, &tie_total);
  int keeps = 0;
  for (int i = i0, tr = tie_rank; i < i1; ++i) {
    const uint32_t u = keys[i];
    if (u > theta) ++keeps;
    else if (u == theta) keeps += (tr++ < need);
  }
  int keep_total;
  int pos = block_excl_scan(keeps, scratch, &keep_total);
  for (int i = i0, tr = tie_rank; i < i1; ++i) {
    const uint32_t u = keys[i];
    const bool keep = u > theta || (u == theta && tr++ < need);
    if (keep) s[pos++] = composite(u, idx ? idx[i] : i);
  }
  __syncthreads();
}

struct FinalizeParams {
  int rows, C, topk, n_q, n_k, pos_offset;
  const uint32_t* cand_key;
  const int32_t* cand_idx;
  const int32_t* cand_cnt;
  const uint32_t* full_keys;  // decode: [rows, n_k] keys for the overflow path
  int32_t* out_idx;
  float* out_scores;
};

__device__ void write_sorted(const FinalizeParams& p, int r, const uint64_t* s, int n_sorted) {
  int32_t* oi = p.out_idx + (size_t)r * p.topk;
  float* os = p.out_scores ? p.out_scores + (size_t)r * p.topk : nullptr;
  for (int i = threadIdx.x; i < p.topk; i += blockDim.x) {
    const bool v = i < n_sorted;
    const uint64_t c = v ? s[i] : 0ull;
    oi[i] = v ? (int32_t)(~(uint32_t)c) : -1;
    if (os) os[i] = v ? key_score((uint32_t)(c >> 32)) : -__builtin_inff();
  }
}

__device__ void pad_and_sort(uint64_t* s, int n_items) {
  int n = 1;
  while (n < n_items) n <<= 1;
  for (int i = n_items + threadIdx.x; i < n; i += blockDim.x) s[i] = 0ull;
  __syncthreads();
  block_bitonic_desc(s, n);
}

// Prefill rows: each candidate list (<= kPrefillMaxC entries, in index order)
// is a superset of the row's top-k. The exact k-th key is found in LDS, the k
// winners are collected in list order (ties: lowest index) and sorted.
constexpr int kPrefillMaxC = 8192;
constexpr int kMaxTopk = 2048;

__global__ __launch_bounds__(kFinNT) void prefill_finalize_kernel(FinalizeParams p) {
  __shared__ uint32_t skey[kPrefillMaxC];
  __shared__ uint64_t s[kMaxTopk];
  __shared__ uint32_t hist[256];
  __shared__ int scratch[17];
  const int r = blockIdx.x;
  const int t = r % p.n_q;
  const int n_valid = min(p.pos_offset + t + 1, p.n_k);
  const int k_eff = min(p.topk, n_valid);
  const int cnt = min(p.cand_cnt[r], p.C);  // >= k_eff by construction
  const uint32_t* ck = p.cand_key + (size_t)r * p.C;
  const int32_t* ci = p.cand_idx + (size_t)r * p.C;
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) skey[i] = ck[i];
  __syncthreads();
  uint32_t theta = 0u;
  int need = 1 << 30;
  const int take = min(k_eff, cnt);
  if (cnt > take) block_kth_key(skey, cnt, take, hist, &theta, &need);
  block_ordered_collect(skey, ci, cnt, theta, need, s, scratch);
  pad_and_sort(s, take);
  write_sorted(p, r, s, take);
}

// Decode requests: the candidate list (unordered, <= C = kFinMax entries) is
// sorted whole; if it overflowed, the exact top-k is taken from the request's
// full key row instead.
__global__ __launch_bounds__(kFinNT) void decode_finalize_kernel(FinalizeParams p) {
  __shared__ uint64_t s[kFinMax];
  __shared__ uint32_t hist[256];
  __shared__ int scratch[17];
  const int r = blockIdx.x;
  const int t = r % p.n_q;
  const int n_valid = min(p.pos_offset + t + 1, p.n_k);
  const int k_eff = min(p.topk, n_valid);
  const int cnt = p.cand_cnt[r];
  int n_sorted;
  if (cnt <= p.C) {
    const uint32_t* ck = p.cand_key + (size_t)r * p.C;
    const int32_t* ci = p.cand_idx + (size_t)r * p.C;
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) s[i] = composite(ck[i], ci[i]);
    pad_and_sort(s, cnt);
    n_sorted = min(cnt, k_eff);
  } else {
    const uint32_t* keys = p.full_keys + (size_t)r * p.n_k;
    uint32_t theta;
    int need;
    block_kth_key(keys, n_valid, k_eff, hist, &theta, &need);
    block_ordered_collect(keys, nullptr, n_valid, theta, need, s, scratch);
    pad_and_sort(s, k_eff);
    n_sorted = k_eff;
  }
  write_sorted(p, r, s, n_sorted);
}

hipError_t launch_topk_finalize(const IndexerParams& ip, int rows, hipStream_t s) {
  FinalizeParams p;
  p.rows = rows;
  p.C = ip.C;
  p.topk = ip.topk;
  p.n_q = ip.n_q;
  p.n_k = ip.n_k;
  p.pos_offset = ip.pos_offset;
  p.cand_key = ip.cand_key;
  p.cand_idx = ip.cand_idx;
  p.cand_cnt = ip.cand_cnt;
  p.full_keys = ip.dec_keys;
  p.out_idx = ip.out_idx;
  p.out_scores = ip.out_scores;
  if (ip.n_q == 1)
    hipLaunchKernelGGL(decode_finalize_kernel, dim3(rows), dim3(kFinNT), 0, s, p);
  else
    hipLaunchKernelGGL(prefill_finalize_kernel, dim3(rows), dim3(kFinNT), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- decode path

__global__ void fill_u32_kernel(uint32_t* __restrict__ a, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    a[i] = v;
}

// One query (64 heads max) against 256 keys per workgroup, 64 per wave; the
// k rows stream straight from HBM into MFMA B-fragments (each row is used
// once). Writes each causal key's 32-bit order key and adds the block's
// histogram of the top kDecodeHistBits bits to the request's global histogram.
template <int D, int MB, bool FP8, bool DUMP>
__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerParams p) {
  constexpr int KS = FP8 ? D / 64 : D / 16;
  constexpr int RB = FP8 ? D : 2 * D;  // bytes per key row
  __shared__ uint32_t hist[kDecodeHistBins];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int i32 = lane & 31, g = lane >> 5;
  const size_t row = (size_t)b * p.n_q;  // n_q == 1
  const int kend = min(p.pos_offset + 1, p.n_k);
  const int base = blockIdx.x * kDecodeKeysPerBlock + wave * kWave;

  for (int i = threadIdx.x; i < kDecodeHistBins; i += blockDim.x) hist[i] = 0u;

  typedef typename std::conditional<FP8, i32x8, bf16x8>::type Frag;
  Frag qa[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = 32 * mb + i32;
    const bool ok = head < p.H;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (FP8) {
        i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ok) {
          const unsigned char* src = (const unsigned char*)p.q + (row * p.H + head) * D + g * (D / 2) + 32 * ks;
          const i32x4 lo = *(const i32x4*)src, hi = *(const i32x4*)(src + 16);
          v = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        qa[mb][ks] = v;
      } else {
        bf16x8 v = {};
        if (ok) v = *(const bf16x8*)((const __bf16*)p.q + (row * p.H + head) * D + g * (D / 2) + 8 * ks);
        qa[mb][ks] = v;
      }
    }
  }
  float wr[MB][16];
  const float qs = FP8 ? p.q_scale[row] : 1.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
      wr[mb][r] = head < p.H ? p.w[row * p.H + head] * qs : 0.0f;
    }

  // B fragments straight from global memory
  Frag kb[2][KS];
  const unsigned char* kbase = (const unsigned char*)p.k + (size_t)b * p.n_k * RB;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int key = base + 32 * nb + i32;
    const bool ok = key < kend;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (FP8) {
        i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ok) {
          const unsigned char* src = kbase + (size_t)key * RB + g * (D / 2) + 32 * ks;
          const i32x4 lo = *(const i32x4*)src, hi = *(const i32x4*)(src + 16);
          v = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        kb[nb][ks] = v;
      } else {
        bf16x8 v = {};
        if (ok) v = *(const bf16x8*)(kbase + (size_t)key * RB + 2 * (g * (D / 2) + 8 * ks));
        kb[nb][ks] = v;
      }
    }
  }
  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (FP8)
          acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][ks], kb[nb][ks], acc[mb][nb],
                                                                       0, 0, 0, 127, 0, 127);
        else
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb[nb][ks], acc[mb][nb], 0, 0, 0);
      }
  float part[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    float s = 0.0f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s = __builtin_fmaf(wr[mb][r], fmaxf(acc[mb][nb][r], 0.0f), s);
    part[nb] = s;
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                   false, false);
  float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  const int key = base + lane;
  const bool valid = key < kend;
  if constexpr (FP8) score *= valid ? p.k_scale[(size_t)b * p.n_k + key] : 0.0f;
  const uint32_t u = score_key(score);
  if (valid) {
    p.dec_keys[(size_t)b * p.n_k + key] = u;
    if constexpr (DUMP) p.dump[row * (size_t)p.n_k + key] = canon_zero(score);
  }
  __syncthreads();
  if (valid) atomicAdd(&hist[u >> (32 - kDecodeHistBits)], 1u);
  __syncthreads();
  uint32_t* gh = p.dec_hist + (size_t)b * kDecodeHistBins;
  for (int i = threadIdx.x; i < kDecodeHistBins; i += blockDim.x) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Threshold bin of one request: the largest bin T with
// count(bins >= T) >= k_eff. Computed by one wave.
__device__ int wave_threshold_bin(const uint32_t* __restrict__ gh, int k_eff) {
  constexpr int PER = kDecodeHistBins / kWave;
  const int lane = lane_id();
  const int top = kDecodeHistBins - 1 - PER * lane;  // lane l owns bins top .. top-PER+1
  uint32_t loc = 0;
  for (int j = 0; j < PER; ++j) loc += gh[top - j];
  const uint32_t incl = wave_incl_scan(loc);
  const uint64_t m = ballot(incl >= (uint32_t)k_eff);
  const int L = uniform_i(m ? __builtin_ctzll(m) : 63);
  int bin = 0;
  if (lane == L) {
    uint32_t cum = incl - loc;
    bin = top - PER + 1;
    for (int j = 0; j < PER; ++j) {
      cum += gh[top - j];
      if (cum >= (uint32_t)k_eff) {
        bin = top - j;
        break;
      }
    }
  }
  return __builtin_amdgcn_readlane(bin, L);
}

// Appends every key whose top bits reach the threshold bin to the request's
// candidate list (count may exceed C: the finalize kernel then falls back to
// an exact full-row select).
__global__ __launch_bounds__(256) void decode_collect_kernel(IndexerParams p) {
  __shared__ int sh_bin;
  const int b = blockIdx.y;
  const int n_valid = min(p.pos_offset + 1, p.n_k);
  const int k_eff = min(p.topk, n_valid);
  if (threadIdx.x < kWave) {
    const int bin = wave_threshold_bin(p.dec_hist + (size_t)b * kDecodeHistBins, k_eff);
    if (threadIdx.x == 0) sh_bin = bin;
  }
  __syncthreads();
  const uint32_t tbin = (uint32_t)sh_bin;
  const int chunk = (n_valid + gridDim.x - 1) / gridDim.x;
  const int beg = blockIdx.x * chunk, end = min(beg + chunk, n_valid);
  const uint32_t* keys = p.dec_keys + (size_t)b * p.n_k;
  uint32_t* ck = p.cand_key + (size_t)b * p.C;
  int32_t* ci = p.cand_idx + (size_t)b * p.C;
  for (int i0 = beg; i0 < end; i0 += blockDim.x) {
    const int i = i0 + threadIdx.x;
    const bool in = i < end;
    const uint32_t u = in ? keys[i] : 0u;
    const bool sel = in && (u >> (32 - kDecodeHistBits)) >= tbin;
    const uint64_t m = ballot(sel);
    if (m) {
      int basepos = 0;
      if (lane_id() == 0) basepos = atomicAdd(&p.cand_cnt[b], popc64(m));
      basepos = __shfl(basepos, 0, 64);
      const int pos = basepos + mbcnt(m);
      if (sel && pos < p.C) {
        ck[pos] = u;
        ci[pos] = i;
      }
    }
  }
}

template <int D, int MB, bool FP8>
static void launch_decode_scores_t(const IndexerParams& p, hipStream_t s) {
  const dim3 grid((p.n_k + kDecodeKeysPerBlock - 1) / kDecodeKeysPerBlock, p.B);
  if (p.dump)
    hipLaunchKernelGGL((indexer_decode_kernel<D, MB, FP8, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((indexer_decode_kernel<D, MB, FP8, false>), grid, dim3(256), 0, s, p);
}

hipError_t launch_indexer_decode(const IndexerParams& p, hipStream_t s) {
  // zero the histograms and candidate counters (a fill kernel, not a memset node)
  const size_t nh = (size_t)p.B * kDecodeHistBins;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((nh + 255) / 256)), dim3(256), 0, s, p.dec_hist, nh, 0u);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((p.B + 255) / 256)), dim3(256), 0, s,
                     (uint32_t*)p.cand_cnt, (size_t)p.B, 0u);
  hipError_t e = record_phase(p.ev, 0, s);
  if (e != hipSuccess) return e;
  const bool two = p.H > 32;
  if (p.fp8) {
    if (p.D == 64) two ? launch_decode_scores_t<64, 2, true>(p, s) : launch_decode_scores_t<64, 1, true>(p, s);
    else two ? launch_decode_scores_t<128, 2, true>(p, s) : launch_decode_scores_t<128, 1, true>(p, s);
  } else {
    if (p.D == 32) two ? launch_decode_scores_t<32, 2, false>(p, s) : launch_decode_scores_t<32, 1, false>(p, s);
    else if (p.D == 64) two ? launch_decode_scores_t<64, 2, false>(p, s) : launch_decode_scores_t<64, 1, false>(p, s);
    else two ? launch_decode_scores_t<128, 2, false>(p, s) : launch_decode_scores_t<128, 1, false>(p, s);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = record_phase(p.ev, 1, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_collect_kernel, dim3(kDecodeCollectBlocks, p.B), dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_topk_finalize(p, p.B, s);
  if (e != hipSuccess) return e;
  return record_phase(p.ev, 2, s);
}

}  // namespace dsa
