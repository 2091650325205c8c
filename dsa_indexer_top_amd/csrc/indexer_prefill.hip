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
// theta is a lower bound of the k-th largest 32-bit order key seen so far,
// chosen so that at least k listed entries are >= theta (0 before the first
// shrink). A new key is appended iff its key > theta: a later key that only
// ties theta ranks below those k entries because it has a higher index. When
// the list is nearly full, a wave-level radix select shrinks it (see
// wave_shrink), keeping the list in index order and a superset of the top-k.
// The finalize kernel then sorts each row's <= C survivors.
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

// Radix-select step over one 8-bit digit of the keys whose bits above `shift+8`
// equal `prefix` (under `pmask`): builds the 256-bin histogram in `hist` (LDS
// of this wave) reading the list 8 keys per lane per batch, then returns the
// digit d holding the rem-th largest such key and the number of such keys
// with a digit above d (via *above) and in d (via *in_d).
__device__ __forceinline__ int wave_digit_step(const uint32_t* __restrict__ keys, int cnt, uint32_t prefix,
                                               uint32_t pmask, int shift, uint32_t rem, uint32_t* hist,
                                               uint32_t* above, uint32_t* in_d) {
  const int lane = lane_id();
  for (int i = lane; i < 256; i += kWave) hist[i] = 0u;
  wave_sync();
  for (int base = 0; base < cnt; base += 8 * kWave) {
    uint32_t u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kWave + lane;
      u[j] = i < cnt ? keys[i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kWave + lane;
      if (i < cnt && (u[j] & pmask) == prefix) atomicAdd(&hist[(u[j] >> shift) & 255u], 1u);
    }
  }
  wave_sync();
  // lane l owns digits 255-4l .. 252-4l, so lane order is descending digit order
  const int hb = 255 - 4 * lane;
  const uint32_t c0 = hist[hb], c1 = hist[hb - 1], c2 = hist[hb - 2], c3 = hist[hb - 3];
  const uint32_t loc = c0 + c1 + c2 + c3;
  const uint32_t incl = wave_incl_scan(loc);
  const uint64_t m = ballot(incl >= rem);
  const int L = uniform_i(m ? __builtin_ctzll(m) : 63);
  const uint32_t cum = incl - loc;
  int digit;
  uint32_t ab, in;
  if (cum + c0 >= rem) {
    digit = hb; ab = cum; in = c0;
  } else if (cum + c0 + c1 >= rem) {
    digit = hb - 1; ab = cum + c0; in = c1;
  } else if (cum + c0 + c1 + c2 >= rem) {
    digit = hb - 2; ab = cum + c0 + c1; in = c2;
  } else {
    digit = hb - 3; ab = cum + c0 + c1 + c2; in = c3;
  }
  *above = (uint32_t)__builtin_amdgcn_readlane((int)ab, L);
  *in_d = (uint32_t)__builtin_amdgcn_readlane((int)in, L);
  wave_sync();
  return __builtin_amdgcn_readlane(digit, L);
}

// Stable in-place compaction of the first `cnt` entries: keeps every key
// > theta and the first `ties_left` keys == theta, in list order. Returns the
// new count.
__device__ __forceinline__ int wave_compact_keep(uint32_t* __restrict__ keys, int32_t* __restrict__ idxs,
                                                 int cnt, uint32_t theta, int ties_left) {
  const int lane = lane_id();
  int out = 0, ties = 0;
  for (int base = 0; base < cnt; base += 8 * kWave) {
    uint32_t u[8];
    int32_t s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * kWave + lane;
      u[j] = i < cnt ? keys[i] : 0u;
      s[j] = i < cnt ? idxs[i] : 0;
    }
    // every write of this batch lands at or below the chunk being processed,
    // and the whole batch was read above
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = base + j * kWave + lane < cnt;
      const bool tie = in && u[j] == theta;
      const uint64_t tm = ballot(tie);
      const bool keep = in && (u[j] > theta || (tie && ties + mbcnt(tm) < ties_left));
      ties += popc64(tm);
      const uint64_t km = ballot(keep);
      if (keep) {
        const int o = out + mbcnt(km);
        keys[o] = u[j];
        idxs[o] = s[j];
      }
      out += popc64(km);
    }
  }
  wave_sync();
  return out;
}

// Shrinks one row's candidate list (cnt > k entries, all of keys earlier than
// any future arrival) so that it still holds the row's top-k, and returns the
// new acceptance threshold: a later key is kept iff its key is > threshold.
// Fast path: two 8-bit digit steps find the 16-bit prefix P of the k-th largest
// key; at least k listed keys are >= theta = P<<16, so a later key <= theta
// ranks below k earlier ones (ties go to the lower index) and can be dropped,
// and the list keeps its keys >= theta (k plus the few sharing prefix P).
// If that keeps too many (heavy ties), two more digit steps give the exact
// k-th key theta and the list keeps exactly k entries: those > theta and the
// lowest-index ties (the list is in index order).
__device__ __noinline__ uint32_t wave_shrink(uint32_t* __restrict__ keys, int32_t* __restrict__ idxs,
                                             int* cnt_io, int k, int keep_max, uint32_t* hist) {
  const int cnt = *cnt_io;
  wave_sync();
  uint32_t above, in_d;
  uint32_t rem = (uint32_t)k;
  const int d1 = wave_digit_step(keys, cnt, 0u, 0u, 24, rem, hist, &above, &in_d);
  rem -= above;
  uint32_t prefix = (uint32_t)d1 << 24;
  const int d2 = wave_digit_step(keys, cnt, prefix, 0xFF000000u, 16, rem, hist, &above, &in_d);
  rem -= above;
  prefix |= (uint32_t)d2 << 16;
  const uint32_t kept = (uint32_t)k - rem + in_d;  // keys with prefix >= P
  if ((int)kept <= keep_max) {
    *cnt_io = wave_compact_keep(keys, idxs, cnt, prefix, 1 << 30);
    return prefix;
  }
  const int d3 = wave_digit_step(keys, cnt, prefix, 0xFFFF0000u, 8, rem, hist, &above, &in_d);
  rem -= above;
  prefix |= (uint32_t)d3 << 8;
  const int d4 = wave_digit_step(keys, cnt, prefix, 0xFFFFFF00u, 0, rem, hist, &above, &in_d);
  rem -= above;
  prefix |= (uint32_t)d4;
  *cnt_io = wave_compact_keep(keys, idxs, cnt, prefix, (int)rem);
  return prefix;
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
  // Two register stages: the fetch of tile t+2 is issued right after the
  // barrier that publishes tile t+1 and only stored to LDS one full iteration
  // later, so L2/MALL latency hides behind a whole tile of MFMA work.
  i32x4 stage0[CPT], stage1[CPT];
  const unsigned char* kbase = (const unsigned char*)p.k + (size_t)b * p.n_k * T::kRowBytes;
  int ld_row[CPT], ld_goff[CPT], ld_soff[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * NT;
    const int r = ch / T::kChunksPerRow, col = ch % T::kChunksPerRow;
    ld_row[c] = ch < T::kChunks ? r : (1 << 30);
    ld_goff[c] = r * T::kRowBytes + col * 16;
    ld_soff[c] = r * T::kLdsRow + col * 16;
  }
  auto load_tile = [&](i32x4 (&st)[CPT], int tile) {
    const unsigned char* src = kbase + (size_t)tile * kTileKeys * T::kRowBytes;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      i32x4 v = {0, 0, 0, 0};
      if (tile * kTileKeys + ld_row[c] < p.n_k) v = *(const i32x4*)(src + ld_goff[c]);
      st[c] = v;
    }
  };
  auto store_tile = [&](const i32x4 (&st)[CPT], int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (ld_row[c] < kTileKeys) *(i32x4*)(&lds_k[buf][ld_soff[c]]) = st[c];
  };

  uint32_t theta = 0u;
  int cnt = 0;
  uint32_t* ckey = p.cand_key + row * (size_t)p.C;
  int32_t* cidx = p.cand_idx + row * (size_t)p.C;
  const float* kscale = FP8 ? p.k_scale + (size_t)b * p.n_k : nullptr;

  // One 32-key half tile (N block nb of LDS tile kt): the MFMAs into `acc`,
  // interleaved k-step by k-step with the epilogue of the previous half `prev`
  // (ReLU as an integer max on the float bits, since negative floats and -0.0
  // have negative bit patterns; then the head weights and the head sum). Each
  // k-step chunk is fenced with sched_barrier so that one wave keeps both the
  // matrix core and the VALU busy; B fragments are read two k-steps ahead.
  // Returns this lane's partial score of key (lane & 31) of the previous half
  // over its 16 * MB heads (0 when EPI is false).
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type BFrag;
  constexpr int EPK = (16 * MB + KS - 1) / KS;  // epilogue elements per k-step
  auto read_b = [&](const unsigned char* src0, int ks) -> BFrag {
    if constexpr (FP8) {
      const unsigned char* src = src0 + g * (D / 2) + 32 * ks;
      const i32x4 lo = *(const i32x4*)src;
      const i32x4 hi = *(const i32x4*)(src + 16);
      return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return *(const bf16x8*)(src0 + g * D + 16 * ks);
    }
  };
  auto half_step = [&](auto EPI_T, auto MMA_T, const unsigned char* kt, int nb, f32x16 (&acc)[MB],
                       const f32x16 (&prev)[MB]) -> float {
    constexpr bool EPI = decltype(EPI_T)::value;
    constexpr bool MMA = decltype(MMA_T)::value;
    const unsigned char* src0 = kt + (32 * nb + i32) * T::kLdsRow;
    BFrag bf[3];
    if constexpr (MMA) {
      bf[0] = read_b(src0, 0);
      if (KS > 1) bf[1 % 3] = read_b(src0, KS > 1 ? 1 : 0);
    }
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (MMA) {
        if (ks + 2 < KS) bf[(ks + 2) % 3] = read_b(src0, ks + 2);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if constexpr (FP8)
            acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                qa[mb][ks], bf[ks % 3], ks == 0 ? f32x16{} : acc[mb], 0, 0, 0, 127, 0, 127);
          else
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], bf[ks % 3],
                                                               ks == 0 ? f32x16{} : acc[mb], 0, 0, 0);
        }
      }
      if constexpr (EPI) {
#pragma unroll
        for (int e = ks * EPK; e < (ks + 1) * EPK && e < 16 * MB; ++e) {
          const float x = __int_as_float(max(__float_as_int(prev[e >> 4][e & 15]), 0));
          if (e & 1) s1 = __builtin_fmaf(wr[e >> 4][e & 15], x, s1);
          else s0 = __builtin_fmaf(wr[e >> 4][e & 15], x, s0);
        }
        // keep this chunk's epilogue inside the chunk (IR passes would
        // otherwise sink it below every fence)
        asm volatile("" : "+v"(s0), "+v"(s1));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return s0 + s1;
  };
  using TrueT = std::integral_constant<bool, true>;
  using FalseT = std::integral_constant<bool, false>;
  // Join the two half-tile partials (v_permlane32_swap: lane l < 32 gets key l
  // of half 0, lane l >= 32 key l of half 1), then the streaming filter.
  auto finish_tile = [&](int base, float part0, float part1, float ksc) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part0), __float_as_uint(part1),
                                                     false, false);
    float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int key = base + lane;
    const bool valid = key < kend;
    if constexpr (FP8) score *= ksc;
    if constexpr (DUMP) {
      if (valid) p.dump[row * (size_t)p.n_k + key] = canon_zero(score);
    }
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
        theta = uniform_u(wave_shrink(ckey, cidx, &cnt, p.topk, p.C - 2 * kTileKeys, lds_hist[wave]));
        cnt = uniform_i(cnt);
      }
    }
  };

  f32x16 accA[MB], accB[MB];
  if (n_tiles > 0) {
    load_tile(stage0, 0);
    store_tile(stage0, 0);
  }
  if (n_tiles > 1) load_tile(stage1, 1);
  // Nothing may stay in flight into the loop: the loop's own prefetches are
  // then the only outstanding loads the MFMAs could be made to wait for.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (kend > 0) half_step(FalseT{}, TrueT{}, lds_k[0], 0, accA, accB);
  // One tile: second half-tile of `tile` (+ epilogue of its first half), then
  // publish tile+1 (held in st_next) and start fetching tile+2 into st_free,
  // then the first half of tile+1 (+ epilogue of tile's second half).
  auto iteration = [&](int tile, const i32x4 (&st_next)[CPT], i32x4 (&st_free)[CPT]) {
    const int cur = tile & 1;
    const bool more = tile + 1 < n_tiles;
    const int base = tile * kTileKeys;
    const bool mine = base < kend;                          // wave-uniform
    const bool mine_next = more && base + kTileKeys < kend;
    float ksc = 1.0f;
    if constexpr (FP8) ksc = (mine && base + lane < kend) ? kscale[base + lane] : 0.0f;
    float part0 = 0.0f, part1 = 0.0f;
    if (mine) part0 = half_step(TrueT{}, TrueT{}, lds_k[cur], 1, accB, accA);
    if (more) store_tile(st_next, cur ^ 1);
    __syncthreads();
    if (tile + 2 < n_tiles) load_tile(st_free, tile + 2);
    if (mine) {
      if (mine_next)
        part1 = half_step(TrueT{}, TrueT{}, lds_k[cur ^ 1], 0, accA, accB);
      else
        part1 = half_step(TrueT{}, FalseT{}, lds_k[cur], 0, accA, accB);
      finish_tile(base, part0, part1, ksc);
    }
  };
  for (int tile = 0; tile < n_tiles; tile += 2) {
    iteration(tile, stage1, stage0);
    if (tile + 1 < n_tiles) iteration(tile + 1, stage0, stage1);
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
