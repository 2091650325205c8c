// Prefill lightning indexer fused with a streaming per-row top-k filter.
//
// Computes, for every query t and causal key s <= pos(t):
//     I[t,s] = sum_j w'[t,j] * ReLU(q[t,j,:] . k[s,:]) * kscale[s]
// (bf16: w' = w, kscale = 1; fp8: w' = w * q_scale[t], kscale = k_scale[s];
// ReLU(a*x) = a*ReLU(x) for a > 0 lets the per-token scales leave the dot
// product), and keeps, per query row, a candidate list that provably contains
// the row's top-k. The score matrix only ever lives in registers.
//
// Mapping (gfx950, wave64). A workgroup owns 4 consecutive query rows, one per
// wave. A wave holds its row's indexer queries as MFMA A-fragments in
// registers (heads are the M dimension, padded to 32 or 64 rows) and streams
// k through double-buffered, padded LDS, 128 keys per loop iteration (keys are
// the N dimension, head_dim the K dimension). v_mfma_f32_32x32x16_bf16 (fp8:
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

// Waves (query rows) per workgroup: 4, so two workgroups share a CU and one
// can run its MFMAs while the other waits at its per-tile barrier (the K tile
// goes straight to LDS, so a smaller workgroup costs no staging registers).
template <bool FP8>
constexpr int prefill_waves() { return 4; }
constexpr int kMaxPrefillWaves = 8;
constexpr int kTileKeys = 64;                  // keys per LDS sub-tile and per filter commit
constexpr int kIterKeys = 2 * kTileKeys;       // keys per loop iteration (one barrier)
// Appends a list may receive between the commit that flags it as nearly full
// and the shrink that serves the flag: the flagging commit and the next one,
// 128 keys each.
constexpr int kListMargin = 4 * kTileKeys;

template <int D, bool FP8>
struct KTile {
  static constexpr int kRowBytes = FP8 ? D : 2 * D;
  static constexpr int kChunksPerRow = kRowBytes / 16;
  // +16 bytes per row: the 16-byte reads of 16 consecutive rows hit 16
  // distinct groups of 4 LDS banks, and a row's fragment reads are immediate
  // offsets from its address. A direct load fills 64 consecutive 16-byte
  // slots; lanes whose slot is a row's padding load nothing.
  static constexpr int kLdsRow = kRowBytes + 16;
  static constexpr int kSlotsPerRow = kChunksPerRow + 1;
  static constexpr int kSlots = kTileKeys * kSlotsPerRow;
  static constexpr int kBytes = kTileKeys * kLdsRow;
};

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (the LDS address must be the same for the whole wave). A
// plain device function: the host pass cannot see this builtin inside the
// kernel's lambdas.
__device__ __forceinline__ void lds_load16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// Workgroup-shared scratch of the cooperative list shrink.
constexpr int kShrinkHistCopies = 8;  // interleaved copies: clustered keys would serialise one copy

struct ShrinkLds {
  uint32_t hist[256 * kShrinkHistCopies];
  int scan[kMaxPrefillWaves + 1];
  int res[4];                       // digit, keys above the digit, keys in the digit
  uint32_t flags[3];                // bit w: the row of wave w needs a shrink (iteration mod 3)
  int cnt[kMaxPrefillWaves];        // that row's list length (in), new length (out)
  uint32_t theta[kMaxPrefillWaves]; // new acceptance threshold (out)
};

// Exclusive prefix sum over the workgroup (one value per thread, list order =
// thread order); *total = sum. Contains barriers: call from every thread.
template <int W>
__device__ int coop_excl_scan(int v, ShrinkLds& sh, int* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan((uint32_t)v);
  if (lane == 63) sh.scan[wave] = (int)incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int x = sh.scan[w];
    before += w < wave ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + (int)incl - v;
}

// A shrink reads the list in rounds of 8 entries per thread, each thread
// taking 8 consecutive entries with two 16-byte loads: a round covers 2048
// entries (four rounds for C = 8192), so a pass over the list costs four
// memory round trips. (16 entries per thread would halve that again but push
// the kernel's registers past 256.)
constexpr int kShrinkPerThread = 8;

// Loads the list entries of this thread in the round starting at `base`
// (entries at or past cnt read as 0). cnt <= C and C is a multiple of 64, so a
// 16-byte quad that starts below cnt lies inside the row's list.
// The loads are unconditional, clamped into the row's list (cap = C entries);
// the masking is arithmetic, so no per-entry condition mask is kept live.
template <typename T>
__device__ __forceinline__ void load_round(const T* __restrict__ src, int base, int cnt, int cap,
                                           T (&v)[kShrinkPerThread]) {
  const int i0 = base + (int)threadIdx.x * kShrinkPerThread;
#pragma unroll
  for (int q = 0; q < kShrinkPerThread / 4; ++q) {
    const i32x4 x = *(const i32x4*)(src + min(i0 + 4 * q, cap - 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int m = (i0 + 4 * q + e - cnt) >> 31;  // all ones below cnt
      asm volatile("" : "+v"(m));             // kept as a lane mask, not a condition
      v[4 * q + e] = (T)(x[e] & m);
    }
  }
}

// One radix-select step over an 8-bit digit of the listed keys whose higher
// bits match `prefix` under `pmask`: the whole workgroup builds the 256-bin
// histogram, wave 0 finds the digit holding the rem-th largest such key.
// Returns the digit; *above / *in_d = matching keys with a larger digit /
// with this digit. Entries past cnt read as key 0, which lies below every
// score's key and so below the selected digit.
template <int W>
__device__ int coop_digit_step(const uint32_t* __restrict__ keys, int cnt, int cap, uint32_t prefix, uint32_t pmask,
                               int shift, uint32_t rem, ShrinkLds& sh, uint32_t* above, uint32_t* in_d) {
  constexpr int NT = W * kWave;
  for (int i = threadIdx.x; i < 256 * kShrinkHistCopies; i += NT) sh.hist[i] = 0u;
  __syncthreads();
  const uint32_t copy = threadIdx.x % kShrinkHistCopies;
#pragma unroll 1
  for (int base = 0; base < cnt; base += kShrinkPerThread * NT) {
    uint32_t u[kShrinkPerThread];
    load_round(keys, base, cnt, cap, u);
#pragma unroll
    for (int j = 0; j < kShrinkPerThread; ++j) {
      if ((u[j] & pmask) == prefix) atomicAdd(&sh.hist[((u[j] >> shift) & 255u) * kShrinkHistCopies + copy], 1u);
      __builtin_amdgcn_sched_barrier(0);  // one entry's condition at a time
    }
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int hb = 255 - 4 * lane;  // lane order = descending digit order
    uint32_t c0 = 0u, c1 = 0u, c2 = 0u, c3 = 0u;
#pragma unroll
    for (int j = 0; j < kShrinkHistCopies; ++j) {
      c0 += sh.hist[hb * kShrinkHistCopies + j];
      c1 += sh.hist[(hb - 1) * kShrinkHistCopies + j];
      c2 += sh.hist[(hb - 2) * kShrinkHistCopies + j];
      c3 += sh.hist[(hb - 3) * kShrinkHistCopies + j];
    }
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
    if (lane == L) {
      sh.res[0] = digit;
      sh.res[1] = (int)ab;
      sh.res[2] = (int)in;
    }
  }
  __syncthreads();
  *above = (uint32_t)sh.res[1];
  *in_d = (uint32_t)sh.res[2];
  const int d = sh.res[0];
  __syncthreads();
  return d;
}

// Ordered in-place compaction by the workgroup: keeps every key > theta and
// the first `ties_left` keys == theta, in list order; returns the new length.
// Each thread owns consecutive entries of a round; all of a round is read
// before any of it is written (the scans hold barriers), and a round only
// writes below its own end. Entries past cnt read as key 0 and are never
// kept (theta is above 0: it is a kept key's prefix, and every score's key
// is at least 2^23).
template <int W>
__device__ int coop_compact(uint32_t* __restrict__ keys, int32_t* __restrict__ idxs, int cnt, int cap, uint32_t theta,
                            int ties_left, ShrinkLds& sh) {
  constexpr int NT = W * kWave;
  constexpr int E = kShrinkPerThread;
  int out = 0, ties = 0;
#pragma unroll 1
  for (int base = 0; base < cnt; base += E * NT) {
    uint32_t u[E];
    int32_t s[E];
    load_round(keys, base, cnt, cap, u);
    load_round(idxs, base, cnt, cap, s);
    int nt = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      nt += u[j] == theta ? 1 : 0;
      __builtin_amdgcn_sched_barrier(0);
    }
    int tie_total;
    int tr = ties + coop_excl_scan<W>(nt, sh, &tie_total);
    uint32_t keep = 0u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const bool eq = u[j] == theta;
      const bool kj = u[j] > theta || (eq && tr < ties_left);
      tr += eq ? 1 : 0;
      keep |= kj ? (1u << j) : 0u;
      __builtin_amdgcn_sched_barrier(0);
    }
    int keep_total;
    int pos = out + coop_excl_scan<W>(__popc(keep), sh, &keep_total);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if ((keep >> j) & 1u) {
        keys[pos] = u[j];
        idxs[pos] = s[j];
        ++pos;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    out += keep_total;
    ties += tie_total;
    __syncthreads();
  }
  return out;
}

// Shrinks one row's candidate list (cnt > k entries, all of keys earlier than
// any future arrival) so that it still holds the row's top-k; run by the whole
// workgroup. Returns the new acceptance threshold (a later key is kept iff
// its key is > threshold) and the new length.
// Fast path: two 8-bit digit steps find the 16-bit prefix P of the k-th largest
// key; at least k listed keys are >= theta = P<<16, so a later key <= theta
// ranks below k earlier ones (ties go to the lower index) and can be dropped,
// and the list keeps its keys >= theta (k plus the few sharing prefix P).
// If that keeps too many (heavy ties), two more digit steps give the exact
// k-th key theta and the list keeps exactly k entries: those > theta and the
// lowest-index ties (the list is in index order).
template <int W>
__device__ __forceinline__ void coop_shrink(uint32_t* __restrict__ keys, int32_t* __restrict__ idxs, int cnt, int cap,
                                            int k, int keep_max, ShrinkLds& sh, uint32_t* theta_out, int* cnt_out) {
  uint32_t prefix = 0u, pmask = 0u;
  uint32_t rem = (uint32_t)k;
  int ties_left = 1 << 30;
#pragma unroll 1
  for (int st = 0; st < 4; ++st) {
    uint32_t above, in_d;
    const int shift = 24 - 8 * st;
    const int d = coop_digit_step<W>(keys, cnt, cap, prefix, pmask, shift, rem, sh, &above, &in_d);
    rem -= above;
    prefix |= (uint32_t)d << shift;
    pmask |= 0xFFu << shift;
    if (st == 1 && (int)((uint32_t)k - rem + in_d) <= keep_max) break;  // keys with prefix >= P fit
    if (st == 3) ties_left = (int)rem;
  }
  const int n = coop_compact<W>(keys, idxs, cnt, cap, prefix, ties_left, sh);
  if (threadIdx.x == 0) {
    *theta_out = prefix;
    *cnt_out = n;
  }
}

template <int D, int MB, bool FP8, bool DUMP>
__global__ __launch_bounds__(prefill_waves<FP8>() * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void indexer_prefill_kernel(IndexerParams p) {
  constexpr int kPrefillWaves = prefill_waves<FP8>();
  using T = KTile<D, FP8>;
  constexpr int NT = kPrefillWaves * kWave;
  constexpr int KS = FP8 ? D / 64 : D / 16;  // MFMA k-steps over head_dim
  constexpr int CPT = (T::kSlots + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][2 * T::kBytes];
  __shared__ ShrinkLds shl;

  const int lane = lane_id();
  const int wave = uniform_i(threadIdx.x >> 6);  // wave-uniform: row state lives in SGPRs
  // a range the compiler cannot see: folds the per-wave guards of the tile
  // loads (1% fewer cycles; lane_id carries the lane's range)
  __builtin_assume(wave >= 0 && wave < kPrefillWaves);
  const int nqb = (p.n_q + kPrefillWaves - 1) / kPrefillWaves;
  const int qb = nqb - 1 - (int)blockIdx.x;  // longest rows first
  const int b = blockIdx.y;
  const int t = qb * kPrefillWaves + wave;
  const bool active = t < p.n_q;
  const size_t row = (size_t)b * p.n_q + (active ? t : 0);
  const int t_last = min(qb * kPrefillWaves + kPrefillWaves, p.n_q) - 1;
  const int kend_wg = min(p.pos_offset + t_last + 1, p.n_k);
  const int kend = active ? min(p.pos_offset + t + 1, p.n_k) : 0;
  const int n_tiles = (kend_wg + kIterKeys - 1) / kIterKeys;
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

  // ---- K tile staging: global -> LDS directly (global_load_lds_dwordx4).
  // Tile t lives in lds_k[t & 1]; it is read in the second half of iteration
  // t - 1 and the first half of iteration t, so its buffer is free after the
  // barrier of iteration t, when the load of tile t + 2 is issued; the wait
  // before the barrier of iteration t + 1 completes it, a whole tile of MFMA
  // work later. No registers hold the tile on the way.
  const unsigned char* kbase = (const unsigned char*)p.k + (size_t)b * p.n_k * T::kRowBytes;
  // The lane offsets of this wave's 16-byte slots inside a full tile are
  // fixed for the whole row and kept in registers, two 16-bit offsets per
  // register (a lane whose slot is a row's padding loads that row's first
  // chunk into the padding, which is never read), so a full tile's load is a
  // scalar base plus a 32-bit lane offset: no 64-bit address math and no
  // exec-mask branch per instruction. The epilogue leaves little VALU time.
  static_assert(T::kSlots % kWave == 0, "a load instruction is all slots or none");
  uint32_t voff[(CPT + 1) / 2];  // two 16-bit offsets per register (a tile is < 64 KB)
#pragma unroll
  for (int c = 0; c < (CPT + 1) / 2; ++c) voff[c] = 0u;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int q = c * NT + wave * kWave + lane;
    const int r = q / T::kSlotsPerRow;
    const int col = q - r * T::kSlotsPerRow;
    voff[c / 2] |= (uint32_t)(r * T::kRowBytes + 16 * (col < T::kChunksPerRow ? col : 0)) << (16 * (c & 1));
  }
  auto dma_sub = [&](int sub, unsigned char* dst) {
    const unsigned char* src = kbase + (size_t)sub * kTileKeys * T::kRowBytes;
    const int rows_left = p.n_k - sub * kTileKeys;
    if (rows_left <= 0) return;  // wholly past n_k: never a valid key
    if (rows_left >= kTileKeys) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int q0 = c * NT + wave * kWave;  // first 16-byte LDS slot of this wave's load (uniform)
        if (q0 < T::kSlots) {
          // extracted here, not hoisted: the load then takes it as a 32-bit
          // offset to the scalar base
          uint32_t o = (voff[c / 2] >> (16 * (c & 1))) & 0xFFFFu;
          asm volatile("" : "+v"(o));
          lds_load16(src + o, dst + 16 * q0);
        }
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q0 = c * NT + wave * kWave;  // first 16-byte LDS slot of this wave's load (uniform)
      if (q0 < T::kSlots) {
        const int q = q0 + lane;
        const int r = q / T::kSlotsPerRow;
        const int col = q - r * T::kSlotsPerRow;
        const int rr = r < rows_left ? r : rows_left - 1;  // rows past n_k repeat the last (masked later)
        if (col < T::kChunksPerRow && r < kTileKeys)
          lds_load16(src + (size_t)rr * T::kRowBytes + 16 * col, dst + 16 * q0);
      }
    }
  };

  // an iteration's tile is two sub-tiles, back to back in one buffer
  auto dma_tile = [&](int tile, int buf) {
    dma_sub(2 * tile, lds_k[buf]);
    dma_sub(2 * tile + 1, lds_k[buf] + T::kBytes);
  };
  // The loads of a whole tile (both sub-tiles full), spread over the KS
  // chunks of a half tile: load i of the 2 * CPT goes with chunk
  // i * KS / (2 * CPT), so a wave never issues its tile share in one burst
  // (the workgroup's waves would queue on the vector memory path together,
  // right after the barrier, and stall their next MFMAs).
  auto dma_full_part = [&](int tile, int buf, int ks) {
#pragma unroll
    for (int i = 0; i < 2 * CPT; ++i) {
      if (min(KS - 1, i * KS / (2 * CPT)) != ks) continue;
      const int sub = i / CPT, c = i % CPT;
      const int q0 = c * NT + wave * kWave;  // first 16-byte LDS slot of this wave's load (uniform)
      if (q0 < T::kSlots) {
        const unsigned char* src = kbase + (size_t)(2 * tile + sub) * kTileKeys * T::kRowBytes;
        uint32_t o = (voff[c / 2] >> (16 * (c & 1))) & 0xFFFFu;
        asm volatile("" : "+v"(o));
        lds_load16(src + o, lds_k[buf] + sub * T::kBytes + 16 * q0);
      }
    }
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
  // With two k-steps per half (fp8), a half can take its B fragments from
  // `pre` (PIN) and read the next half's (tile nkt, block nnb) into it after
  // its first MFMAs (POUT); halves separated by the tile barrier do not.
  // Returns this lane's partial score of key (lane & 31) of the previous half
  // over its 16 * MB heads (0 when EPI is false).
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type BFrag;
  constexpr int EPK = (16 * MB + KS - 1) / KS;  // epilogue elements per k-step
  // B fragment of row r (key), k-step ks: dims g*(D/2) + (8 bf16 | 32 fp8)*ks ..
  auto read_b = [&](const unsigned char* kt, int r, int ks) -> BFrag {
    const unsigned char* row = kt + r * T::kLdsRow;
    if constexpr (FP8) {
      const unsigned char* src = row + g * (D / 2) + 32 * ks;
      const i32x4 lo = *(const i32x4*)src;
      const i32x4 hi = *(const i32x4*)(src + 16);
      return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return *(const bf16x8*)(row + g * D + 16 * ks);
    }
  };

  constexpr int SIDE_KS = KS > 1 ? 1 : 0;  // chunk that also carries the previous tile's filter
  // fp8 (two k-steps per half): the next half's B fragments are read during
  // this half (after its first MFMAs), so its MFMAs need not wait for LDS
  constexpr bool kPre = FP8 && KS == 2;
  BFrag pre[2];
  auto half_step = [&](auto EPI_T, auto MMA_T, auto PIN_T, auto POUT_T, const unsigned char* kt, int nb,
                       const unsigned char* nkt, int nnb, f32x16 (&acc)[MB], const f32x16 (&prev)[MB],
                       auto&& side) -> float {
    constexpr bool EPI = decltype(EPI_T)::value;
    constexpr bool MMA = decltype(MMA_T)::value;
    constexpr bool PIN = decltype(PIN_T)::value && kPre && MMA;
    constexpr bool POUT = decltype(POUT_T)::value && kPre && MMA;
    const int brow = 32 * nb + i32;
    BFrag bf[3];
    if constexpr (PIN) {
      bf[0] = pre[0];
      bf[1] = pre[1];
    } else if constexpr (MMA) {
      bf[0] = read_b(kt, brow, 0);
      if (KS > 1) bf[1 % 3] = read_b(kt, brow, KS > 1 ? 1 : 0);
    }
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (MMA) {
        if (ks + 2 < KS) bf[(ks + 2) % 3] = read_b(kt, brow, ks + 2);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if constexpr (FP8)
            acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                qa[mb][ks], bf[ks % 3], ks == 0 ? f32x16{} : acc[mb], 0, 0, 0, 127, 0, 127);
          else
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], bf[ks % 3],
                                                               ks == 0 ? f32x16{} : acc[mb], 0, 0, 0);
        }
        if constexpr (POUT) {
          if (ks == 0) {
            pre[0] = read_b(nkt, 32 * nnb + i32, 0);
            pre[1] = read_b(nkt, 32 * nnb + i32, 1);
          }
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
      side(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
    return s0 + s1;
  };
  using TrueT = std::integral_constant<bool, true>;
  using FalseT = std::integral_constant<bool, false>;
  // Streaming filter, 64 keys (two half tiles) at a time. filter_compute runs
  // inside a chunk of a later half tile, so its dependency chain (join the
  // two half-tile partials with v_permlane32_swap: lane l < 32 gets key l of
  // half 0, lane l >= 32 key l of half 1) hides behind MFMAs. filter_commit,
  // once per iteration after the barrier, compares both pending groups of 64
  // (the previous tile's keys 64..127, then this tile's 0..63) with the
  // threshold, appends the accepted keys in key order and, when the list is
  // nearly full, flags it for a shrink. With nothing pending, an end of 0
  // makes every lane of that group invalid.
  float pend_p0 = 0.0f, pend_p1 = 0.0f, pend_ksc = 1.0f;
  int pend_base = 0, pend_end = 0;
  float f_score = 0.0f;
  // the previous tile's keys 64..127, computed during the first quarter and
  // committed with this tile's keys 0..63 after the barrier
  float f_score_a = 0.0f;
  int pend_a_base = 0, pend_a_end = 0;
  // theta as a float: the order key is strictly monotone on scores, so
  // key > theta  <=>  score > key_score(theta) (and -inf accepts all).
  float theta_f = -__builtin_inff();
  auto filter_compute = [&]() {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pend_p0), __float_as_uint(pend_p1),
                                                     false, false);
    float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    // never -0 after this (fp8: fma with +0; bf16: + 0), so the commit can
    // take the order key without its -0 case
    score = FP8 ? __builtin_fmaf(score, pend_ksc, 0.0f) : score + 0.0f;
    f_score = score;
    asm volatile("" : "+v"(f_score));
  };
  auto filter_compute_a = [&]() {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pend_p0), __float_as_uint(pend_p1),
                                                     false, false);
    float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    // never -0 after this (fp8: fma with +0; bf16: + 0), so the commit can
    // take the order key without its -0 case
    score = FP8 ? __builtin_fmaf(score, pend_ksc, 0.0f) : score + 0.0f;
    f_score_a = score;
    asm volatile("" : "+v"(f_score_a));
  };
  // par: the iteration mod 3; a full list raises flag bit `wave` of
  // flags[par], which the workgroup reads after the next barrier and serves.
  auto filter_commit = [&](int par) {
    const int key_a = pend_a_base + lane, key = pend_base + lane;
    const bool valid_a = key_a < pend_a_end, valid = key < pend_end;
    if constexpr (DUMP) {
      if (valid_a) p.dump[row * (size_t)p.n_k + key_a] = canon_zero(f_score_a);
      if (valid) p.dump[row * (size_t)p.n_k + key] = canon_zero(f_score);
    }
    const bool take_a = valid_a && f_score_a > theta_f, take = valid && f_score > theta_f;
    // a ballot of one compare is that compare's lane mask (a ballot of the
    // combined condition would go through a VGPR)
    const uint64_t am_a = ballot(valid_a) & ballot(f_score_a > theta_f);
    const uint64_t am = ballot(valid) & ballot(f_score > theta_f);
    if (am_a | am) {
      // list order = key order: the previous tile's keys first
      // 32-bit byte offsets from the row's (scalar) list bases: no 64-bit address math
      if (take_a) {
        const uint32_t off = 4u * (uint32_t)(cnt + mbcnt(am_a));
        *(uint32_t*)((unsigned char*)ckey + off) = score_key_nz(f_score_a);
        *(int32_t*)((unsigned char*)cidx + off) = key_a;
      }
      const int cnt_b = cnt + popc64(am_a);
      if (take) {
        const uint32_t off = 4u * (uint32_t)(cnt_b + mbcnt(am));
        *(uint32_t*)((unsigned char*)ckey + off) = score_key_nz(f_score);
        *(int32_t*)((unsigned char*)cidx + off) = key;
      }
      cnt = cnt_b + popc64(am);
      if (cnt > p.C - kListMargin && lane == 0) atomicOr(&shl.flags[par], 1u << wave);
    }
    pend_a_end = 0;
    pend_end = 0;
  };
  // Called by the whole workgroup with the flags word it read after the
  // barrier: shrinks every flagged row, one at a time; each flagged wave picks
  // up its new threshold and length; the word is cleared for its next use.
  auto coop_shrinks = [&](uint32_t flags, int par) {
    if (flags == 0u) return;
    if (lane == 0) shl.cnt[wave] = cnt;  // current lengths (a commit may have followed the flag)
    __syncthreads();
#pragma unroll 1
    for (int w = 0; w < kPrefillWaves; ++w) {
      if (!((flags >> w) & 1u) || shl.cnt[w] <= p.C - kListMargin) continue;
      const size_t rw = (size_t)b * p.n_q + qb * kPrefillWaves + w;
      coop_shrink<kPrefillWaves>(p.cand_key + rw * p.C, p.cand_idx + rw * p.C, shl.cnt[w], p.C, p.topk, p.C - kListMargin, shl,
                  &shl.theta[w], &shl.cnt[w]);
      __syncthreads();
    }
    if (((flags >> wave) & 1u) && cnt > p.C - kListMargin) {
      theta = uniform_u(shl.theta[wave]);
      theta_f = key_score(theta);
      cnt = uniform_i(shl.cnt[wave]);
    }
    __syncthreads();
    if (threadIdx.x == 0) shl.flags[par] = 0u;
    __syncthreads();
  };
  auto no_side = [&](int) {};
  // callbacks run inside a chunk of a half tile: `f` once, at chunk SIDE_KS
  auto at_side = [&](auto&& f) { return [&f](int ks) { if (ks == SIDE_KS) f(); }; };

  f32x16 accA[MB], accB[MB];
  if (n_tiles > 0) dma_tile(0, 0);
  if (n_tiles > 1) dma_tile(1, 1);
  if (threadIdx.x == 0) {
    shl.flags[0] = 0u;
    shl.flags[1] = 0u;
    shl.flags[2] = 0u;
  }
  // Nothing may stay in flight into the loop: the loop's own prefetches are
  // then the only outstanding loads the MFMAs could be made to wait for.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (kend > 0) half_step(FalseT{}, TrueT{}, FalseT{}, TrueT{}, lds_k[0], 0, lds_k[0], 1, accA, accB, no_side);
  // One iteration, tile = 128 keys in four 32-key quarters q0..q3 (q0 was
  // multiplied in the previous iteration): q1 (+ epilogue of q0, + the filter
  // of the previous tile's keys 64..127), q2 (+ epilogue of q1), q3
  // (+ epilogue of q2, + the filter of keys 0..63), the barrier that
  // publishes tile+1, the commit of both filtered groups, the load of tile+2
  // into the buffer `tile` leaves, and q0 of tile+1 (+ epilogue of q3). Keys
  // 64..127 are then pending for the filter.
  auto iteration = [&](int tile) {
    const int cur = tile & 1;
    const bool more = tile + 1 < n_tiles;
    const int base = tile * kIterKeys;
    const bool mine = base < kend;                          // wave-uniform
    const bool mine_next = more && base + kIterKeys < kend;
    float ksc0 = 1.0f, ksc1 = 1.0f;
    if constexpr (FP8) {
      // unconditional loads, clamped into the row's n_k scales (no exec-mask
      // branch); keys past kend get scale 0
      const int i0 = base + lane, i1 = base + kTileKeys + lane;
      const float s0 = *(const float*)((const char*)kscale + 4u * (uint32_t)min(i0, p.n_k - 1));
      const float s1 = *(const float*)((const char*)kscale + 4u * (uint32_t)min(i1, p.n_k - 1));
      ksc0 = (mine && i0 < kend) ? s0 : 0.0f;
      ksc1 = (mine && i1 < kend) ? s1 : 0.0f;
    }
    // Flag words rotate over three iterations: iteration t's commit (after its
    // barrier) writes word t % 3, iteration t+1 reads it after its own barrier
    // and serves it, and every wave has read it before barrier t+2. (Two
    // words would do since every commit follows a barrier; the third keeps
    // a written word apart from any being read with room to spare.)
    const int par = tile % 3, prev = (tile + 2) % 3;
    float q0 = 0.0f, q1 = 0.0f, q2 = 0.0f, q3 = 0.0f;
    if (mine)
      q0 = half_step(TrueT{}, TrueT{}, TrueT{}, TrueT{}, lds_k[cur], 1, lds_k[cur], 2, accB, accA,
                     at_side(filter_compute_a));
    else filter_compute_a();
    if (mine) {
      q1 = half_step(TrueT{}, TrueT{}, TrueT{}, TrueT{}, lds_k[cur], 2, lds_k[cur], 3, accA, accB, no_side);
      pend_p0 = q0;
      pend_p1 = q1;
      pend_ksc = ksc0;
      pend_base = base;
      pend_end = kend;
      q2 = half_step(TrueT{}, TrueT{}, TrueT{}, FalseT{}, lds_k[cur], 3, lds_k[cur], 0, accB, accA,
                     at_side(filter_compute));
    } else {
      filter_compute();
    }
    // this wave's load of tile+1 (issued one iteration ago) must have landed
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    filter_commit(par);  // the previous tile's keys 64..127 and this tile's 0..63
    // The flags raised by the previous iteration's commits are visible now;
    // read them during the next quarter and serve them after it (the word is
    // next written two iterations later, after the next barrier).
    uint32_t flags_v = 0u;
    auto read_flags = [&]() { flags_v = shl.flags[prev]; };
    // Tile+2 goes into the buffer this tile leaves (every wave has read it:
    // the barrier above). A whole tile's loads are spread over this half
    // tile's chunks; a ragged last tile, or a wave without a half tile to
    // compute, issues them at once.
    const int dtile = tile + 2;
    const bool do_dma = dtile < n_tiles;
    const bool spread = do_dma && mine && (2 * dtile + 2) * kTileKeys <= p.n_k;
    if (do_dma && !spread) dma_tile(dtile, cur);
    auto q3_side = [&](int ks) {
      if (ks == SIDE_KS) read_flags();
      if (spread) dma_full_part(dtile, cur, ks);
    };
    if (mine) {
      if (mine_next)
        q3 = half_step(TrueT{}, TrueT{}, FalseT{}, TrueT{}, lds_k[cur ^ 1], 0, lds_k[cur ^ 1], 1, accA, accB,
                       q3_side);
      else
        q3 = half_step(TrueT{}, FalseT{}, FalseT{}, FalseT{}, lds_k[cur], 0, lds_k[cur], 0, accA, accB,
                       q3_side);
      pend_p0 = q2;
      pend_p1 = q3;
      pend_ksc = ksc1;
      pend_a_base = base + kTileKeys;
      pend_a_end = kend;
    } else {
      read_flags();
    }
    coop_shrinks(uniform_u(flags_v), prev);
  };
  for (int tile = 0; tile < n_tiles; ++tile) iteration(tile);
  filter_compute_a();
  __syncthreads();
  filter_commit(n_tiles % 3);
  __syncthreads();
  coop_shrinks(uniform_u(shl.flags[(n_tiles + 2) % 3]), (n_tiles + 2) % 3);
  coop_shrinks(uniform_u(shl.flags[n_tiles % 3]), n_tiles % 3);
  if (active && lane == 0) p.cand_cnt[row] = cnt;
}

template <int D, int MB, bool FP8>
static hipError_t launch_prefill_t(const IndexerParams& p, hipStream_t s) {
  constexpr int W = prefill_waves<FP8>();
  const dim3 grid((p.n_q + W - 1) / W, p.B);
  const dim3 block(W * kWave);
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
