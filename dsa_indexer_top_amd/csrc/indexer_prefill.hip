// Prefill lightning indexer fused with a streaming per-row top-k filter.
//
// Computes, for every query t and causal key s <= pos(t):
//     I[t,s] = sum_j w'[t,j] * ReLU(q[t,j,:] . k[s,:]) * kscale[s]
// (bf16: w' = w, kscale = 1; fp8: w' = w * q_scale[t], kscale = k_scale[s];
// ReLU(a*x) = a*ReLU(x) for a > 0 lets the per-token scales leave the dot
// product), and keeps, per query row, a candidate list that provably contains
// the row's top-k. The score matrix only ever lives in registers.
//
// Mapping (gfx950, wave64). A workgroup owns 8 consecutive query rows, one per
// wave. A wave holds its row's indexer queries as MFMA A-fragments in
// registers (heads are the M dimension, padded to 32 or 64 rows) and streams
// 64-key tiles of k through double-buffered, padded LDS (keys are the N
// dimension, head_dim the K dimension). v_mfma_f32_32x32x16_bf16 (fp8:
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales) produces a 32 heads x 32
// keys block per lane group; in that layout a lane holds 16 heads of one key,
// so ReLU, the head weights and the head sum are per-lane FMAs, and one
// v_permlane32_swap joins the two half-waves: lane l ends with the score of
// key tile_base + l.
//
// Streaming top-k (per wave = per row). Keys arrive in increasing index order.
// theta is the k-th largest 32-bit order key among the candidates kept so far
// (0 before the first compaction). A new key is appended iff its key > theta:
// a later key that only ties theta ranks below all k kept entries because it
// has a higher index. When the list is nearly full, an exact wave-level radix
// select (4 x 8-bit digits) finds the k-th key and a stable in-place
// compaction keeps exactly the k best (ties by lower index), so the list stays
// in index order. The finalize kernel then sorts each row's <= C survivors.
//
// Workgroups are issued longest row block first to balance the causal
// triangle.
#include "dsa_device.h"
#include "dsa_internal.h"

#include <type_traits>

namespace dsa {

constexpr int kPrefillWaves = 8;
constexpr int kTileKeys = 64;

template <int D, bool FP8>
struct KTile {
  static constexpr int kRowBytes = FP8 ? D : 2 * D;
  // +16 bytes per row: the 16-byte reads of 16 consecutive rows then hit 16
  // distinct groups of 4 LDS banks.
  static constexpr int kLdsRow = kRowBytes + 16;
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kChunks = kTileKeys * kChunksPerRow;
  static constexpr int kBytes = kTileKeys * kLdsRow;
};

// Exact top-k of the first `cnt` (> k) candidates of one row, in place.
// keys/idxs: the row's list (index order). hist: 256 words of LDS owned by the
// wave. Keeps exactly k entries (all keys > theta, then the lowest-index ties
// at theta), in index order, and returns theta = the k-th largest key.
__device__ __noinline__ uint32_t wave_select_compact(uint32_t* __restrict__ keys,
                                                     int32_t* __restrict__ idxs, int cnt, int k,
                                                     uint32_t* hist) {
  const int lane = lane_id();
  wave_sync();
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = lane; i < 256; i += kWave) hist[i] = 0u;
    wave_sync();
    for (int i = lane; i < cnt; i += kWave) {
      const uint32_t u = keys[i];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    wave_sync();
    // lane l owns digits 255-4l .. 252-4l, so lane order is descending digit order
    const int hb = 255 - 4 * lane;
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
    digit = __builtin_amdgcn_readlane(digit, L);
    above = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
    prefix |= (uint32_t)digit << shift;
    pmask |= 0xFFu << shift;
    remaining -= (int)above;
    wave_sync();
  }
  const uint32_t theta = prefix;
  const int need = remaining;  // ties at theta that belong to the top-k
  int out = 0, ties = 0;
  for (int base = 0; base < cnt; base += kWave) {
    const int i = base + lane;
    const bool in = i < cnt;
    const uint32_t u = in ? keys[i] : 0u;
    const int32_t s = in ? idxs[i] : 0;
    const bool tie = in && u == theta;
    const uint64_t tm = ballot(tie);
    const bool keep = in && (u > theta || (tie && ties + mbcnt(tm) < need));
    ties += popc64(tm);
    const uint64_t km = ballot(keep);
    if (keep) {
      const int o = out + mbcnt(km);
      keys[o] = u;
      idxs[o] = s;
    }
    out += popc64(km);
  }
  wave_sync();
  return theta;
}

template <int D, int MB, bool FP8, bool DUMP>
__global__ __launch_bounds__(kPrefillWaves * kWave) void indexer_prefill_kernel(IndexerParams p) {
  using T = KTile<D, FP8>;
  constexpr int NT = kPrefillWaves * kWave;
  constexpr int KS = FP8 ? D / 64 : D / 16;  // MFMA k-steps over head_dim
  constexpr int CPT = (T::kChunks + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][T::kBytes];
  __shared__ uint32_t lds_hist[kPrefillWaves][256];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int nqb = (p.n_q + kPrefillWaves - 1) / kPrefillWaves;
  const int qb = nqb - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const int t = qb * kPrefillWaves + wave;
  const bool active = t < p.n_q;
  const size_t row = (size_t)b * p.n_q + (active ? t : 0);
  const int t_last = min(qb * kPrefillWaves + kPrefillWaves, p.n_q) - 1;
  const int kend_wg = min(p.pos_offset + t_last + 1, p.n_k);
  const int kend = active ? min(p.pos_offset + t + 1, p.n_k) : 0;
  const int n_tiles = (kend_wg + kTileKeys - 1) / kTileKeys;
  const int i32 = lane & 31;
  const int g = lane >> 5;

  // ---- A fragments: this row's indexer queries, heads 32*mb + (lane & 31)
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type AFrag;
  AFrag qa[MB][KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = 32 * mb + i32;
    const bool ok = active && head < p.H;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (FP8) {
        i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ok) {
          const unsigned char* src = (const unsigned char*)p.q + (row * p.H + head) * D +
                                     g * (D / 2) + 32 * ks;
          const i32x4 lo = *(const i32x4*)src;
          const i32x4 hi = *(const i32x4*)(src + 16);
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
  // ---- head weights in the 32x32 accumulator layout: reg r <-> row 8(r/4)+4g+(r%4)
  float wr[MB][16];
  const float qs = (FP8 && active) ? p.q_scale[row] : 1.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
      wr[mb][r] = (active && head < p.H) ? p.w[row * p.H + head] * qs : 0.0f;
    }

  // ---- K tile staging: global -> registers -> LDS
  i32x4 stage[CPT];
  const unsigned char* kbase = (const unsigned char*)p.k + (size_t)b * p.n_k * T::kRowBytes;
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = threadIdx.x + c * NT;
      i32x4 v = {0, 0, 0, 0};
      if (ch < T::kChunks) {
        const int r = ch / T::kChunksPerRow, col = ch % T::kChunksPerRow;
        const int key = tile * kTileKeys + r;
        if (key < p.n_k) v = *(const i32x4*)(kbase + (size_t)key * T::kRowBytes + col * 16);
      }
      stage[c] = v;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = threadIdx.x + c * NT;
      if (ch < T::kChunks) {
        const int r = ch / T::kChunksPerRow, col = ch % T::kChunksPerRow;
        *(i32x4*)(&lds_k[buf][r * T::kLdsRow + col * 16]) = stage[c];
      }
    }
  };

  uint32_t theta = 0u;
  int cnt = 0;
  uint32_t* ckey = p.cand_key + row * (size_t)p.C;
  int32_t* cidx = p.cand_idx + row * (size_t)p.C;
  const float* kscale = FP8 ? p.k_scale + (size_t)b * p.n_k : nullptr;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int cur = tile & 1;
    const bool more = tile + 1 < n_tiles;
    if (more) load_tile(tile + 1);
    const int base = tile * kTileKeys;
    if (base < kend) {
      f32x16 acc[MB][2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;
      const unsigned char* kt = lds_k[cur];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const unsigned char* src = kt + (32 * nb + i32) * T::kLdsRow;
          if constexpr (FP8) {
            src += g * (D / 2) + 32 * ks;
            const i32x4 lo = *(const i32x4*)src;
            const i32x4 hi = *(const i32x4*)(src + 16);
            const i32x8 bf = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  qa[mb][ks], bf, acc[mb][nb], 0, 0, 0, 127, 0, 127);
          } else {
            const bf16x8 bf = *(const bf16x8*)(src + g * D + 16 * ks);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], bf, acc[mb][nb],
                                                                     0, 0, 0);
          }
        }
      }
      // ---- fused epilogue: ReLU, head weights, head sum
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
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                       __float_as_uint(part[1]), false, false);
      float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int key = base + lane;
      const bool valid = key < kend;
      if constexpr (FP8) score *= valid ? kscale[key] : 0.0f;
      if constexpr (DUMP) {
        if (valid) p.dump[row * (size_t)p.n_k + key] = canon_zero(score);
      }
      // ---- streaming filter
      const uint32_t u = score_key(score);
      const bool accept = valid && u > theta;
      const uint64_t am = ballot(accept);
      if (am) {
        if (accept) {
          const int pos = cnt + mbcnt(am);
          ckey[pos] = u;
          cidx[pos] = key;
        }
        cnt += popc64(am);
        if (cnt > p.C - kTileKeys) {
          theta = uniform_u(wave_select_compact(ckey, cidx, cnt, p.topk, lds_hist[wave]));
          cnt = p.topk;
        }
      }
    }
    if (more) store_tile(cur ^ 1);
    __syncthreads();
  }
  if (active && lane == 0) p.cand_cnt[row] = cnt;
}

template <int D, int MB, bool FP8>
static hipError_t launch_prefill_t(const IndexerParams& p, hipStream_t s) {
  const dim3 grid((p.n_q + kPrefillWaves - 1) / kPrefillWaves, p.B);
  const dim3 block(kPrefillWaves * kWave);
  if (p.dump)
    hipLaunchKernelGGL((indexer_prefill_kernel<D, MB, FP8, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((indexer_prefill_kernel<D, MB, FP8, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_topk_finalize(const IndexerParams& p, int rows, hipStream_t s);

hipError_t launch_indexer_prefill(const IndexerParams& p, hipStream_t s) {
  hipError_t e = record_phase(p.ev, 0, s);
  if (e != hipSuccess) return e;
  e = hipErrorInvalidValue;
  const bool two = p.H > 32;
  if (p.fp8) {
    if (p.D == 64) e = two ? launch_prefill_t<64, 2, true>(p, s) : launch_prefill_t<64, 1, true>(p, s);
    else if (p.D == 128) e = two ? launch_prefill_t<128, 2, true>(p, s) : launch_prefill_t<128, 1, true>(p, s);
  } else {
    if (p.D == 32) e = two ? launch_prefill_t<32, 2, false>(p, s) : launch_prefill_t<32, 1, false>(p, s);
    else if (p.D == 64) e = two ? launch_prefill_t<64, 2, false>(p, s) : launch_prefill_t<64, 1, false>(p, s);
    else if (p.D == 128) e = two ? launch_prefill_t<128, 2, false>(p, s) : launch_prefill_t<128, 1, false>(p, s);
  }
  if (e != hipSuccess) return e;
  e = record_phase(p.ev, 1, s);
  if (e != hipSuccess) return e;
  e = launch_topk_finalize(p, p.B * p.n_q, s);
  if (e != hipSuccess) return e;
  return record_phase(p.ev, 2, s);
}

}  // namespace dsa
