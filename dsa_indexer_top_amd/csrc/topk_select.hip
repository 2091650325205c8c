// Exact per-row top-k finalisation and the decode-path selection kernels.
//
// Order used everywhere: higher score first and, for equal scores, lower index
// first (the 32-bit order key score_key(score), then the index ascending).
// The pairs (key, index) are unique, so "the first k in that order" is exactly
// the top-k with the library's tie rule.
#include "dsa_device.h"
#include "dsa_internal.h"

#include <algorithm>
#include <type_traits>

namespace dsa {

// Threads per finalize workgroup (prefill: one per query row, decode: one per
// request): the 8 waves of the radix sort below.
constexpr int kFinNTPrefill = 512;
constexpr int kFinNTDecode = 512;

// Block-wide exclusive prefix sum of one value per thread (blockDim.x <= 1024):
// each wave posts its total, then every wave adds up the totals before it.
__device__ int block_excl_scan(int v, int* scratch /* >= 16 ints */, int* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t incl = wave_incl_scan((uint32_t)v);
  if (lane == 63) scratch[wave] = (int)incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = scratch[w];
    before += w < wave ? x : 0;
    all += x;
  }
  *total = all;
  __syncthreads();  // scratch is free for the next call
  return before + (int)incl - v;
}

// The k-th largest of the keys of the participating entries i < n (get(i, u)
// returns whether entry i takes part and sets its key u; 1 <= k <= their
// count), by 4 radix steps of 8 bits over a 256-bin LDS histogram: *theta =
// that key, *need = how many keys equal to theta belong to the k largest.
// Called by the whole workgroup.
template <class Get>
__device__ void block_kth(Get get, int n, int k, uint32_t* hist, uint32_t* theta, int* need) {
  __shared__ int sh_digit, sh_above;
  uint32_t prefix = 0u, pmask = 0u;
  int remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      uint32_t u;
      if (get(i, u) && (u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
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

// block_kth over every entry of keys[0..n) (LDS or global memory).
__device__ void block_kth_key(const uint32_t* keys, int n, int k, uint32_t* hist, uint32_t* theta,
                              int* need) {
  block_kth([&](int i, uint32_t& u) { u = keys[i]; return true; }, n, k, hist, theta, need);
}

// Emits, in list order, the entries of keys[0..n) that are > theta plus the
// first `need` equal to theta: emit(position, key, token index). idx[i] is
// the token index of entry i (NULL: the entry's position). Each thread owns
// one contiguous segment, so two block-wide scans place every entry.
template <class Emit>
__device__ void block_ordered_emit(const uint32_t* keys, const int32_t* __restrict__ idx, int n, uint32_t theta,
                                   int need, int* scratch, Emit emit) {
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
    if (keep) emit(pos++, u, idx ? idx[i] : i);
  }
  __syncthreads();
}


// Stable LSD radix sort of kSortN (key, index) pairs in LDS by descending key
// (equal keys keep their order) by a workgroup of kSortWaves waves. With
// idx_passes = 2 or 4 (even), that many 8-bit passes by ascending index come
// first, so equal keys end in ascending index order whatever their order was.
// Wave w holds positions 256w + 64j + lane (j < 4) of the current order. Each
// 8-bit pass ranks every element among the equal digits of its wave (lanes
// matched by 8 ballots, rows in order, a per-wave histogram carrying the rows
// before), scans the per-(digit, wave) counts in digit-major order and
// scatters to the other buffer; after the even number of passes the result is
// back in (ka, ia). hist: 256 * kSortWaves entries.
constexpr int kSortWaves = 8;
constexpr int kSortN = kSortWaves * 256;

__device__ void block_radix_sort_desc(uint32_t* ka, int32_t* ia, uint32_t* kb, int32_t* ib, uint32_t* hist,
                                      int* scratch, int idx_passes = 0) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  const uint64_t gt = ~lt & ~(1ull << lane);
  uint32_t* hw = hist + 256 * w;
#pragma unroll 1
  for (int pass = 0; pass < idx_passes + 4; ++pass) {
    const bool by_idx = pass < idx_passes;
    const int shift = 8 * (by_idx ? pass : pass - idx_passes);
    uint32_t u[4], d[4];
    int32_t x[4];
    int rank[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 256 * w + 64 * j + lane;
      u[j] = ka[e];
      x[j] = ia[e];
      // ascending index; ascending ~key = descending key
      d[j] = by_idx ? (((uint32_t)x[j] >> shift) & 255u) : ((~u[j] >> shift) & 255u);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) hw[4 * lane + q] = 0u;
    wave_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint64_t m = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool set = (d[j] >> bit) & 1u;
        const uint64_t bal = ballot(set);
        m &= set ? bal : ~bal;
      }
      rank[j] = (int)hw[d[j]] + popc64(m & lt);
      wave_sync();
      if ((m & gt) == 0ull) hw[d[j]] += (uint32_t)popc64(m);  // the group's highest lane
      wave_sync();
    }
    __syncthreads();
    // thread t owns entries 4t .. 4t+3 of the (digit, wave) order: digit t/2,
    // waves 4(t&1) .. 4(t&1)+3
    const int dg = threadIdx.x >> 1, w0 = 4 * (threadIdx.x & 1);
    uint32_t c[4];
    int tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = hist[256 * (w0 + q) + dg];
      tot += (int)c[q];
    }
    int total;
    int base = block_excl_scan(tot, scratch, &total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hist[256 * (w0 + q) + dg] = (uint32_t)base;
      base += (int)c[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = (int)hist[256 * w + d[j]] + rank[j];
      kb[pos] = u[j];
      ib[pos] = x[j];
    }
    __syncthreads();
    uint32_t* tk = ka; ka = kb; kb = tk;
    int32_t* ti = ia; ia = ib; ib = ti;
  }
}

struct FinalizeParams {
  int rows, C, topk, n_q, n_k, pos_offset;
  const uint32_t* cand_key;
  const int32_t* cand_idx;
  const int32_t* cand_cnt;  // row r at cand_cnt[r * cnt_stride]
  int cnt_stride;
  uint32_t* dec_hist;  // decode: histogram rows, zeroed (with the counter) once read
  const uint32_t* full_keys;  // decode: [rows, decode_key_stride(n_k)] keys for the overflow path
  PagedKV kv;                 // decode: per-request lengths (kv.seq_lens) or none
  int32_t* out_idx;
  float* out_scores;
};

// Writes the first n_sorted sorted pairs of a row, -1 / -inf padded to topk.
__device__ void write_sorted(const FinalizeParams& p, int r, const uint32_t* wkey, const int32_t* widx,
                             int n_sorted) {
  int32_t* oi = p.out_idx + (size_t)r * p.topk;
  float* os = p.out_scores ? p.out_scores + (size_t)r * p.topk : nullptr;
  for (int i = threadIdx.x; i < p.topk; i += blockDim.x) {
    const bool v = i < n_sorted;
    oi[i] = v ? widx[i] : -1;
    if (os) os[i] = v ? key_score(wkey[i]) : -__builtin_inff();
  }
}

// Prefill rows: each candidate list (<= kMaxC entries, in index order)
// is a superset of the row's top-k. Lists without heavy ties are ranked by
// bucket_rank_topk (below); otherwise the exact k-th key is found in LDS, the
// k winners are collected in list order (ties: lowest index) and sorted.
constexpr int kMaxC = 8192;
constexpr int kMaxTopk = 2048;

// Exact top-k of a candidate list (1 <= cnt <= kMaxC entries, distinct
// indices, a superset of the top-k; any order: a prefill row's list is in
// index order, a decode request's is not) by ranking instead of sorting.
// Entries go to 2^kBucketBits buckets by the top bits of (max key - key), so
// that every entry of a lower bucket has a larger key; an LDS counting pass
// returns each entry's slot in its bucket, and an exclusive scan of the counts
// gives each bucket's first rank. Buckets are in rank order, so only the
// prefix up to the end of the bucket holding rank take - 1 can reach the top
// k; those entries store their 64-bit order word (key, ~index) at their slot.
// An entry's rank is its bucket's first rank plus the members of its bucket
// with a larger order word (larger key, or equal key and lower index), and
// entries ranked below `take` are written straight to their output slots. If
// a bucket holds more than kBucketMaxRun entries (heavy ties), it returns
// false before writing any output.
// NARROW: a list longer than 1.5 * take (a prefill row that never filled its
// list and holds every causal key, or one refilled far past take since its
// last shrink) first gets a counting-only pass over the same buckets; the end
// of the bucket holding rank take - 1 bounds the keys that can reach the
// top-k from below, and the ranking pass then buckets only the entries at or
// above that bound, over their own key range. Every other entry ranks below them, so their ranks among themselves
// are the list's ranks. Without it, such a list's 2^kBucketBits buckets span
// its whole key range and crowd the entries around rank take - 1 into a few
// buckets, whose members each compare with the whole bucket.
static_assert(kFinNTPrefill == kFinNTDecode, "one bucket layout for both finalize kernels");
constexpr int kBucketPer = kMaxC / kFinNTDecode;  // entries per thread
constexpr int kBucketEarly = kBucketPer / 2;      // of them loaded before the count is known
constexpr int kBucketMaxRun = 256;
// LDS of the ranking path: the order words, then the bucket counts
constexpr int bucket_lds_bytes(int bits) { return kMaxC * 8 + (4 << bits); }

// Bucket of an order key over the keys [lo, umax]: a lower bucket holds only
// larger keys, and equal keys share a bucket. Keys are log-like in the score
// on either side of zero, so a range on one side is cut into equal key spans,
// (umax - u) >> shift. A range across zero spans the key bits of every tiny
// magnitude in between, which would put all scores of ordinary size into a
// few buckets; there the score itself is cut into equal spans, the rounded
// (smax - s) * inv (monotone in s, clamped to the last bucket).
template <int kBuckets>
struct BucketMap {
  uint32_t umax;
  int shift;
  bool lin;
  float smax, inv;
  // lo and hi are the same in every lane; so is the map (scalar registers)
  __device__ void set(uint32_t lo, uint32_t hi) {
    lo = uniform_u(lo);
    umax = uniform_u(hi);
    shift = (umax - lo) >> __builtin_ctz(kBuckets) ? 32 - __builtin_clz(umax - lo) - __builtin_ctz(kBuckets) : 0;
    smax = key_score(umax);
    const float d = smax - key_score(lo);
    lin = lo < 0x80000000u && umax >= 0x80000000u && d >= 1e-30f && d <= 3e38f;
    inv = __uint_as_float(uniform_u(__float_as_uint(lin ? (float)kBuckets / d : 0.0f)));
  }
  // the range holds more than one bucket's span
  __device__ bool spread() const { return lin || shift > 0; }
  __device__ uint32_t operator()(uint32_t u) const {
    if (lin) return min((uint32_t)((smax - key_score(u)) * inv), (uint32_t)(kBuckets - 1));
    return (umax - u) >> shift;
  }
};

// Entry i = threadIdx.x + e * kFinNTDecode of the list (entries past the
// list's end are ignored).
struct BucketEntries {
  uint32_t u[kBucketPer];
  int32_t x[kBucketPer];
};

__device__ void bucket_load(BucketEntries& v, const uint32_t* __restrict__ ck, const int32_t* __restrict__ ci,
                            int e0, int e1, int lim) {
#pragma unroll
  for (int e = 0; e < kBucketPer; ++e) {
    if (e < e0 || e >= e1) continue;
    const int i = threadIdx.x + e * kFinNTDecode;
    v.u[e] = i < lim ? ck[i] : 0u;
    v.x[e] = i < lim ? ci[i] : 0;
  }
}

template <int kBucketBits, int H, bool NARROW>
__device__ bool bucket_rank_topk(const FinalizeParams& p, int r, const BucketEntries& v, int cnt, int take,
                                 uint64_t* word, uint32_t* base, int* scratch) {
  constexpr int kBuckets = 1 << kBucketBits;
  constexpr int PER = kBucketPer, BPT = kBuckets / kFinNTDecode;  // buckets per thread
  static_assert(BPT * kFinNTDecode == kBuckets && PER * kFinNTDecode == kMaxC, "bucket layout");
  __shared__ uint32_t sh_min[kSortWaves], sh_max[kSortWaves], sh_run[kSortWaves];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (threadIdx.x + e * kFinNTDecode < cnt) {
      mn = min(mn, v.u[e]);
      mx = max(mx, v.u[e]);
    }
  }
#pragma unroll
  for (int q = 0; q < BPT; ++q) base[BPT * threadIdx.x + q] = 0u;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, d, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, d, 64));
  }
  if (lane == 0) {
    sh_min[w] = mn;
    sh_max[w] = mx;
  }
  __syncthreads();
  uint32_t umin = sh_min[0], umax = sh_max[0];
#pragma unroll
  for (int q = 1; q < kSortWaves; ++q) {
    umin = min(umin, sh_min[q]);
    umax = max(umax, sh_max[q]);
  }
  uint32_t lo = umin;  // entries with a key >= lo take part
  BucketMap<kBuckets> map;
  map.set(lo, umax);
  if (NARROW && 2 * cnt > 3 * take && map.spread()) {  // uniform
    __shared__ uint32_t sh_b;
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (threadIdx.x + e * kFinNTDecode < cnt) atomicAdd(&base[map(v.u[e])], 1u);
    __syncthreads();
    uint32_t c[BPT], local = 0u;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      c[q] = base[BPT * threadIdx.x + q];
      local += c[q];
    }
    int all;
    uint32_t pre = (uint32_t)block_excl_scan((int)local, scratch, &all);  // its barriers order the reads above
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (c[q] && pre <= (uint32_t)(take - 1) && (uint32_t)(take - 1) < pre + c[q]) sh_b = BPT * threadIdx.x + q;
      pre += c[q];
      base[BPT * threadIdx.x + q] = 0u;
    }
    __syncthreads();
    const uint32_t bt = sh_b;  // the bucket holding rank take - 1
    if (!map.lin) {
      // the lowest key bucket bt spans (umin if that is below it)
      const uint64_t span = (uint64_t)(bt + 1) << map.shift;
      lo = span > (uint64_t)(umax - umin) ? umin : (uint32_t)(umax - span + 1u);
    } else {
      // the lowest listed key of the buckets up to bt (sh_min is free: the
      // scan's barriers follow its last read)
      uint32_t m = 0xFFFFFFFFu;
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (threadIdx.x + e * kFinNTDecode < cnt && map(v.u[e]) <= bt) m = min(m, v.u[e]);
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) m = min(m, (uint32_t)__shfl_xor((int)m, d, 64));
      if (lane == 0) sh_min[w] = m;
      __syncthreads();
      lo = sh_min[0];
#pragma unroll
      for (int q = 1; q < kSortWaves; ++q) lo = min(lo, sh_min[q]);
    }
    map.set(lo, umax);
  }
  uint32_t slot[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e)
    slot[e] = threadIdx.x + e * kFinNTDecode < cnt && v.u[e] >= lo ? atomicAdd(&base[map(v.u[e])], 1u) : 0u;
  __syncthreads();
  uint32_t c[BPT], local = 0u, run = 0u;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    c[q] = base[BPT * threadIdx.x + q];
    local += c[q];
    run = max(run, c[q]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) run = max(run, (uint32_t)__shfl_xor((int)run, d, 64));
  if (lane == 0) sh_run[w] = run;
  int n_in;  // entries taking part
  uint32_t pre = (uint32_t)block_excl_scan((int)local, scratch, &n_in);  // its barriers order the reads above
  // buckets are laid out in rank order, so the entries that can rank below
  // `take` are the prefix up to the end of the bucket holding rank take - 1
  __shared__ int sh_prefix;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    base[BPT * threadIdx.x + q] = pre;
    if (c[q] && pre <= (uint32_t)(take - 1) && (uint32_t)(take - 1) < pre + c[q]) sh_prefix = (int)(pre + c[q]);
    pre += c[q];
  }
  int max_run = (int)sh_run[0];
#pragma unroll
  for (int q = 1; q < kSortWaves; ++q) max_run = max(max_run, (int)sh_run[q]);  // uniform
  __syncthreads();
  if (max_run > kBucketMaxRun) return false;
  const int prefix = sh_prefix;  // take <= the entries taking part, so one bucket holds rank take - 1
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (threadIdx.x + e * kFinNTDecode < cnt && v.u[e] >= lo) {
      const int s0 = (int)base[map(v.u[e])];
      if (s0 < prefix) word[s0 + slot[e]] = ((uint64_t)v.u[e] << 32) | (uint32_t)~(uint32_t)v.x[e];
    }
  }
  __syncthreads();
  int32_t* oi = p.out_idx + (size_t)r * p.topk;
  float* os = p.out_scores ? p.out_scores + (size_t)r * p.topk : nullptr;
  // One group of H entries per thread at a time: each steps through its
  // bucket with no branch between the LDS reads, so that they are in flight
  // together (a step past the bucket re-reads its last member and is not
  // counted). A list of at most H entries per thread is ranked from the
  // entries in registers (entries past the prefix skipped); a longer one by
  // positions j < prefix of the bucket-ordered words, consecutive positions on
  // consecutive lanes (so a wave's lanes mostly share a bucket).
  auto rank_group = [&](const uint64_t (&mine)[H], const int (&s0)[H], const int (&len)[H]) {
    int rank[H], last[H], wrun = 0;
#pragma unroll
    for (int q = 0; q < H; ++q) {
      rank[q] = s0[q];
      last[q] = s0[q] + max(len[q] - 1, 0);
      wrun = max(wrun, len[q]);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) wrun = max(wrun, __shfl_xor(wrun, d, 64));
    wrun = uniform_i(wrun);
    for (int j = 0; j < wrun; ++j) {
      uint64_t o[H];
#pragma unroll
      for (int q = 0; q < H; ++q) o[q] = word[min(s0[q] + j, last[q])];
#pragma unroll
      for (int q = 0; q < H; ++q) rank[q] += (int)(o[q] > mine[q]) & (int)(j < len[q]);
    }
#pragma unroll
    for (int q = 0; q < H; ++q) {
      if (len[q] > 0 && rank[q] < take) {  // len > 0: an entry of the prefix
        oi[rank[q]] = (int32_t)~(uint32_t)mine[q];
        if (os) os[rank[q]] = key_score((uint32_t)(mine[q] >> 32));
      }
    }
  };
  if (cnt <= H * kFinNTDecode) {
    uint64_t mine[H];
    int s0[H], len[H];
#pragma unroll
    for (int q = 0; q < H; ++q) {
      const bool in = threadIdx.x + q * kFinNTDecode < cnt && v.u[q] >= lo;
      const uint32_t bk = in ? map(v.u[q]) : 0u;
      s0[q] = (int)base[bk];
      len[q] = in && s0[q] < prefix ? (bk + 1 < (uint32_t)kBuckets ? (int)base[bk + 1] : n_in) - s0[q] : 0;
      mine[q] = ((uint64_t)v.u[q] << 32) | (uint32_t)~(uint32_t)v.x[q];
    }
    rank_group(mine, s0, len);
  } else {
    for (int g0 = 0; g0 * kFinNTDecode < prefix; g0 += H) {
      uint64_t mine[H];
      int s0[H], len[H];
#pragma unroll
      for (int q = 0; q < H; ++q) {
        const int j = threadIdx.x + (g0 + q) * kFinNTDecode;
        const bool in = j < prefix;
        mine[q] = word[in ? j : 0];
        const uint32_t bk = map((uint32_t)(mine[q] >> 32));
        s0[q] = (int)base[in ? bk : 0u];
        len[q] = in ? (bk + 1 < (uint32_t)kBuckets ? (int)base[bk + 1] : n_in) - s0[q] : 0;
      }
      rank_group(mine, s0, len);
    }
  }
  for (int i = take + (int)threadIdx.x; i < p.topk; i += blockDim.x) {
    oi[i] = -1;
    if (os) os[i] = -__builtin_inff();
  }
  return true;
}

// two workgroups per CU (4 waves per SIMD: at most 128 VGPRs), so one row's
// barriers and loads overlap another's work
__global__ __launch_bounds__(kFinNTPrefill) __attribute__((amdgpu_waves_per_eu(4))) void prefill_finalize_kernel(
    FinalizeParams p) {
  static_assert(kFinNTPrefill == kSortWaves * kWave && kSortN >= kMaxTopk, "sort layout");
  static_assert(kMaxC >= 2 * kSortN + 256 * kSortWaves, "sort scratch must fit in skey");
  // one LDS buffer (72 KB: two workgroups per CU): the ranking path's words and
  // bucket counts, or the sort path's candidate keys (skey; after the collect,
  // the sort's second buffers and histograms), winners (wkey, widx) and the
  // select histogram
  constexpr int kBits = 11;
  static_assert(kMaxC * 4 + 2 * kSortN * 4 + 256 * 4 <= bucket_lds_bytes(kBits), "sort path fits the buffer");
  __shared__ __attribute__((aligned(16))) unsigned char lds[bucket_lds_bytes(kBits)];
  uint32_t* const skey = (uint32_t*)lds;
  uint32_t* const wkey = skey + kMaxC;
  int32_t* const widx = (int32_t*)(wkey + kSortN);
  uint32_t* const hist = (uint32_t*)(widx + kSortN);
  __shared__ int scratch[17];
  const int r = blockIdx.x;
  const int t = r % p.n_q;
  const int n_valid = min(p.pos_offset + t + 1, p.n_k);
  const int k_eff = min(p.topk, n_valid);
  const uint32_t* ck = p.cand_key + (size_t)r * p.C;
  const int32_t* ci = p.cand_idx + (size_t)r * p.C;
  BucketEntries ent;
  bucket_load(ent, ck, ci, 0, kBucketEarly, min(p.C, kMaxC));
  const int cnt = min(p.cand_cnt[(size_t)r * p.cnt_stride], p.C);  // >= k_eff by construction
  const int take = min(k_eff, cnt);
  if (cnt >= 1) {
    bucket_load(ent, ck, ci, kBucketEarly, kBucketPer, cnt);
    if (bucket_rank_topk<kBits, 4, true>(p, r, ent, cnt, take, (uint64_t*)lds, (uint32_t*)(lds + kMaxC * 8), scratch))
      return;
  }
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) skey[i] = ck[i];
  __syncthreads();
  uint32_t theta = 0u;
  int need = 1 << 30;
  if (cnt > take) block_kth_key(skey, cnt, take, hist, &theta, &need);
  // winners in list order, i.e. index order; padding (key 0) sorts last
  block_ordered_emit(skey, ci, cnt, theta, need, scratch, [&](int pos, uint32_t u, int32_t ix) {
    wkey[pos] = u;
    widx[pos] = ix;
  });
  for (int i = take + (int)threadIdx.x; i < kSortN; i += blockDim.x) {
    wkey[i] = 0u;
    widx[i] = -1;
  }
  __syncthreads();
  // stable by key: equal keys stay in index order, the tie rule
  block_radix_sort_desc(wkey, widx, skey, (int32_t*)(skey + kSortN), skey + 2 * kSortN, scratch);
  write_sorted(p, r, wkey, widx, take);
}

// Decode requests: the candidate list is unordered (<= C entries, a superset
// of the top-k). Lists without heavy ties are ranked by bucket_rank_topk;
// otherwise the k-th key theta is found in LDS; if more entries tie at
// theta than the top-k takes, a second select over their inverted indices
// keeps the lowest ones. The winners (in list order) are radix-sorted by key,
// then each run of equal keys is put in index order (a run longer than 32:
// the row is sorted again with index passes first). If the list overflowed,
// the exact top-k is taken from the request's full key row in index order
// instead, and the stable key sort alone gives the tie rule.
__global__ __launch_bounds__(kFinNTDecode) void decode_finalize_kernel(FinalizeParams p) {
  static_assert(kFinNTDecode == kSortWaves * kWave && kSortN >= kMaxTopk, "sort layout");
  static_assert(kMaxC >= 2 * kSortN + 256 * kSortWaves, "sort scratch must fit in skey");
  args_now((int)blockDim.x, p.kv.seq_lens, p.pos_offset, p.n_k, p.topk, p.C, p.cand_key, p.cand_idx, p.cand_cnt,
           p.cnt_stride, p.dec_hist, p.out_idx, p.out_scores, p.full_keys);
  // one LDS buffer: the bucket path's order words and bucket counts, or the
  // sort path's candidate keys (skey) and winners (wkey, widx)
  constexpr int kBits = 12;  // few workgroups: the finest buckets that fit
  static_assert(kMaxC * 4 + 2 * kSortN * 4 <= bucket_lds_bytes(kBits), "sort path fits the buffer");
  __shared__ __attribute__((aligned(16))) unsigned char lds[bucket_lds_bytes(kBits)];
  uint32_t* const skey = (uint32_t*)lds;
  uint32_t* const wkey = skey + kMaxC;
  int32_t* const widx = (int32_t*)(wkey + kSortN);
  __shared__ uint32_t hist[256];
  __shared__ int scratch[17];
  __shared__ int sh_n;
  const int r = blockIdx.x;  // n_q == 1: row = request
  const int n_valid = decode_len(p.kv, r, p.pos_offset, p.n_k);
  const int k_eff = min(p.topk, n_valid);
  const uint32_t* ck = p.cand_key + (size_t)r * p.C;
  const int32_t* ci = p.cand_idx + (size_t)r * p.C;
  // the list's first entries are loaded together with its count
  BucketEntries ent;
  bucket_load(ent, ck, ci, 0, kBucketEarly, min(p.C, kMaxC));
  // the request's histogram row and counter are left zero for the next
  // decode call on this workspace: the bins are no longer read, the counter
  // once every thread has it
  __shared__ int sh_cnt;
  if (threadIdx.x == 0) sh_cnt = p.cand_cnt[(size_t)r * p.cnt_stride];
  uint32_t* gh = p.dec_hist + (size_t)r * kDecodeHistRow;
  static_assert(kDecodeCntOffset % 4 == 0 && kDecodeHistStride % 4 == 0, "16-byte clears");
  for (int i = threadIdx.x; i < kDecodeHistRow / 4; i += blockDim.x)
    if (i != kDecodeCntOffset / 4) ((uint4*)gh)[i] = make_uint4(0u, 0u, 0u, 0u);  // all but the counter's 16 bytes
  __syncthreads();
  const int cnt = sh_cnt;
  if (threadIdx.x == 0) gh[kDecodeCntOffset] = 0u;
  int take;
  bool ordered;  // winners already in index order
  if (cnt <= p.C) {
    take = min(k_eff, cnt);  // cnt >= k_eff by construction
    if (cnt >= 1) {
      bucket_load(ent, ck, ci, kBucketEarly, kBucketPer, cnt);  // the rest (zeros past the end)
      if (bucket_rank_topk<kBits, 8, false>(p, r, ent, cnt, take, (uint64_t*)lds, (uint32_t*)(lds + kMaxC * 8), scratch))
        return;
    }
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) skey[i] = ck[i];
    if (threadIdx.x == 0) sh_n = 0;
    __syncthreads();
    uint32_t theta = 0u;     // below every finite score's key: keep all
    uint32_t cut = 0u;       // keep ties with ~index >= cut
    if (cnt > take) {
      int need;
      block_kth_key(skey, cnt, take, hist, &theta, &need);
      int ties = 0;
      for (int i = threadIdx.x; i < cnt; i += blockDim.x) ties += skey[i] == theta;
      int tie_total;
      block_excl_scan(ties, scratch, &tie_total);
      if (tie_total > need) {
        int one;
        block_kth([&](int i, uint32_t& u) {
                    u = ~(uint32_t)ci[i];
                    return skey[i] == theta;
                  },
                  cnt, need, hist, &cut, &one);
      }
    }
    for (int i0 = 0; i0 < cnt; i0 += blockDim.x) {
      const int i = i0 + threadIdx.x;
      const uint32_t u = i < cnt ? skey[i] : 0u;
      const int32_t ix = i < cnt ? ci[i] : 0;
      const bool keep = i < cnt && (u > theta || (u == theta && ~(uint32_t)ix >= cut));
      const uint64_t m = ballot(keep);
      int base = 0;
      if (lane_id() == 0 && m) base = atomicAdd(&sh_n, popc64(m));
      base = __shfl(base, 0, 64);
      if (keep) {
        wkey[base + mbcnt(m)] = u;
        widx[base + mbcnt(m)] = ix;
      }
    }
    ordered = false;
  } else {
    const uint32_t* keys = p.full_keys + (size_t)r * decode_key_stride(p.n_k);
    uint32_t theta;
    int need;
    block_kth_key(keys, n_valid, k_eff, hist, &theta, &need);
    block_ordered_emit(keys, nullptr, n_valid, theta, need, scratch, [&](int pos, uint32_t u, int32_t ix) {
      wkey[pos] = u;
      widx[pos] = ix;
    });
    take = k_eff;
    ordered = true;
  }
  // padding (key 0, index -1) sorts last
  for (int i = take + (int)threadIdx.x; i < kSortN; i += blockDim.x) {
    wkey[i] = 0u;
    widx[i] = -1;
  }
  __syncthreads();
  uint32_t* kb = skey;
  int32_t* ib = (int32_t*)(skey + kSortN);
  uint32_t* sh = skey + 2 * kSortN;
  block_radix_sort_desc(wkey, widx, kb, ib, sh, scratch);
  if (!ordered) {
    // equal keys are adjacent now, in list order: the thread at the start of
    // a run puts it in index order (insertion sort); a run longer than 32
    // sends the whole row to a re-sort with index passes first
    bool long_run = false;
    for (int i = threadIdx.x; i + 1 < take; i += blockDim.x) {
      const uint32_t u = wkey[i];
      if ((i > 0 && wkey[i - 1] == u) || wkey[i + 1] != u) continue;  // not the start of a run
      int n = 2;
      while (i + n < take && n <= 32 && wkey[i + n] == u) ++n;
      if (n > 32) {
        long_run = true;
        continue;
      }
      for (int a = i + 1; a < i + n; ++a) {
        const int32_t x = widx[a];
        int c = a - 1;
        while (c >= i && widx[c] > x) {
          widx[c + 1] = widx[c];
          --c;
        }
        widx[c + 1] = x;
      }
    }
    if (__syncthreads_or(long_run))
      block_radix_sort_desc(wkey, widx, kb, ib, sh, scratch, n_valid <= 65536 ? 2 : 4);
  }
  write_sorted(p, r, wkey, widx, take);
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
  p.cnt_stride = ip.cnt_stride;
  p.dec_hist = ip.dec_hist;
  p.full_keys = ip.dec_keys;
  p.kv = ip.kv;
  p.out_idx = ip.out_idx;
  p.out_scores = ip.out_scores;
  if (ip.n_q == 1)
    hipLaunchKernelGGL(decode_finalize_kernel, dim3(rows), dim3(kFinNTDecode), 0, s, p);
  else
    hipLaunchKernelGGL(prefill_finalize_kernel, dim3(rows), dim3(kFinNTPrefill), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- decode path

// Decode set-up: zeroes the histograms and candidate counters (n words from
// p.dec_hist, every block) and, for ragged lengths, block 0 plans the score
// kernel's blocks: request b's keys are cut into 128-key units and each block
// takes up to per = ceil(U / aim) units of one request (U = all requests'
// units, aim = max(target - B, target / 2)). Block j gets (request, k0, k1) in
// dec_work[j]; entries past the last planned block get request -1. The block
// count is at most aim + B <= target + B, since
// sum_b ceil(u_b / per) <= U / per + B.
__global__ __launch_bounds__(256) void decode_prepare_kernel(IndexerParams p, size_t n, int n_work) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p.dec_hist[i] = 0u;
  if (blockIdx.x != 0 || !p.kv.seq_lens) return;
  __shared__ int scratch[17];
  __shared__ unsigned long long sh_units;
  const int per_thread = (p.B + (int)blockDim.x - 1) / (int)blockDim.x;  // requests b0 .. b0 + per_thread - 1
  const int b0 = (int)threadIdx.x * per_thread, b1 = min(b0 + per_thread, p.B);
  if (threadIdx.x == 0) sh_units = 0ull;
  __syncthreads();
  unsigned long long units = 0ull;
  for (int b = b0; b < b1; ++b)
    units += (unsigned long long)((decode_len(p.kv, b, 0, p.n_k) + kDecodeBlockKeys - 1) / kDecodeBlockKeys);
  atomicAdd(&sh_units, units);
  __syncthreads();
  const unsigned long long U = sh_units;
  // aim at target - B blocks so that the rounding up per request still leaves
  // at most target blocks: one even round of a block per CU, no tail
  const unsigned long long aim = (unsigned long long)max(kDecodeTargetBlocks - p.B, kDecodeTargetBlocks / 2);
  const long long per = U == 0ull ? 1ll : (long long)((U + aim - 1) / aim);
  const long long span = per * kDecodeBlockKeys;  // keys per planned block
  int nblk = 0;
  for (int b = b0; b < b1; ++b) nblk += (int)((decode_len(p.kv, b, 0, p.n_k) + span - 1) / span);
  int total;
  int at = block_excl_scan(nblk, scratch, &total);
  for (int b = b0; b < b1; ++b) {
    const int len = decode_len(p.kv, b, 0, p.n_k);
    for (long long k = 0; k < len; k += span, ++at) {
      int32_t* wk = p.dec_work + 3 * (size_t)at;
      wk[0] = b;
      wk[1] = (int)k;
      wk[2] = (int)min((long long)len, k + span);
    }
  }
  for (int j = total + (int)threadIdx.x; j < n_work; j += blockDim.x) p.dec_work[3 * (size_t)j] = -1;
}

// One decode query (up to 64 heads) per request against its key cache. The
// grid is (blocks per request, B); the four waves of a block take 32-key steps
// of the block's key range in turn. A step's k rows are read with fully
// coalesced 16-byte loads (a row's bytes by consecutive lanes) into one of two
// register buffers, written to the wave's LDS tile (rows padded by 16 bytes
// so the fragment reads below are bank-conflict free) and read back as MFMA B
// fragments; the loads of step i + 2 are issued as soon as step i's rows are
// in LDS, so two steps are in flight while the MFMAs and the epilogue run.
// Each causal key's 32-bit order key goes to the workspace; the block's
// histogram of the top kDecodeHistBits bits is kept in LDS and added to the
// request's global histogram once, at the end.
template <int D, bool FP8>
struct DecodeTile {
  static constexpr int RB = FP8 ? D : 2 * D;        // bytes per key row
  static constexpr int RS = RB + 16;                // LDS bytes per row
  static constexpr int LPR = RB / 16;               // lanes per row in a load
  static constexpr int RPI = kWave / LPR;           // rows per load instruction
  static constexpr int NI = kDecodeWaveKeys / RPI;  // load instructions per step
  static constexpr int BYTES = kDecodeWaveKeys * RS;
  static_assert((RS / 16) % 2 == 1, "16-lane phases of a fragment read must cover distinct banks");
};

template <int D, int MB, bool FP8, bool DUMP>
__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerParams p) {
  using T = DecodeTile<D, FP8>;
  const int grid_x = gridDim.x;
  args_now(grid_x, p.q, p.w, p.q_scale, p.k, p.k_scale, p.dec_keys, p.dec_hist, p.dec_work, p.dump, p.kv.seq_lens,
           p.kv.block_table, p.n_q, p.n_k, p.H, p.pos_offset);
  constexpr int KS = FP8 ? D / 64 : D / 16;
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type Frag;
  __shared__ uint32_t hist[kDecodeHistBins];
  __shared__ __attribute__((aligned(16))) unsigned char tile[4][T::BYTES];
  const int lane = lane_id(), wave = uniform_i(threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < 4);
  int b, k0, k1;
  if (p.kv.seq_lens) {
    // ragged lengths: this block's (request, key range) from the device-side plan
    const int32_t* wk = p.dec_work + 3 * (size_t)blockIdx.x;
    b = uniform_i(wk[0]);
    if (b < 0) return;  // whole block: past the planned blocks
    k0 = uniform_i(wk[1]);
    k1 = uniform_i(wk[2]);
  } else {
    // one length for all: gridDim.x blocks split each request's keys evenly
    b = blockIdx.y;
    const int kend = decode_len(p.kv, b, p.pos_offset, p.n_k);
    const int per = ((kend + grid_x - 1) / grid_x + kDecodeBlockKeys - 1) / kDecodeBlockKeys *
                    kDecodeBlockKeys;
    k0 = blockIdx.x * per;
    k1 = min(k0 + per, kend);
  }
  const int i32 = lane & 31, g = lane >> 5;
  const size_t row = (size_t)b * p.n_q;  // n_q == 1

  const bool paged = p.kv.block_table != nullptr;
  const unsigned char* kbase = (const unsigned char*)p.k + (paged ? 0 : (size_t)b * p.n_k * T::RB);
  const float* kscale = FP8 ? p.k_scale + (paged ? 0 : (size_t)b * p.n_k) : nullptr;
  uint32_t* keys_out = p.dec_keys + (size_t)b * decode_key_stride(p.n_k);
  unsigned char* lt = tile[wave];
  const int lr = lane / T::LPR, lc = lane % T::LPR;  // load: row in group, 16-byte chunk

  // Paged: the page ids of this wave's steps are held one per lane (lane j:
  // step pg0 + j) and read with readlane, so a step's row loads never wait on
  // a block-table load (which would also drain the loads of the step before
  // it); the table is re-read once per 64 steps.
  const int wbase = k0 + kDecodeWaveKeys * wave;  // this wave's first step
  int pg = 0, pg0 = -64;
  auto pool_row = [&](int base) -> size_t {
    if (!paged) return (size_t)base;
    const int i = (base - wbase) / kDecodeBlockKeys;  // wave-uniform step number
    if (i - pg0 >= 64) {
      pg0 = i;
      const int kk = base + kDecodeBlockKeys * lane;
      int page = kk < k1 ? p.kv.block_table[(size_t)b * p.kv.max_pages + kk / p.kv.page_size] : 0;
      pg = page < 0 ? 0 : (page >= p.kv.num_pages ? p.kv.num_pages - 1 : page);
    }
    const int page = __builtin_amdgcn_readlane(pg, i - pg0);
    return (size_t)page * p.kv.page_size + base % p.kv.page_size;
  };
  // rows base .. base + 31, coalesced; rows past k1 repeat the step's last
  // valid row (masked later). A step lies inside one page (page_size is a
  // multiple of 32 and steps start at multiples of 32).
  auto load_step = [&](i32x4 (&buf)[T::NI], float& ksc, int base) {
    const size_t r0 = pool_row(base);  // pool row of key `base`
    const int last = k1 - 1 - base;
#pragma unroll
    for (int i = 0; i < T::NI; ++i) {
      const int kr = min(T::RPI * i + lr, last);
      // read once per call: nontemporal, so the stream does not displace the
      // score keys and histograms the next kernels read (8% faster at B = 32)
      buf[i] = __builtin_nontemporal_load((const i32x4*)(kbase + (r0 + kr) * T::RB + 16 * lc));
    }
    if constexpr (FP8) ksc = kscale[r0 + min(i32, last)];
  };
  // the first two steps' rows are requested before anything else, so that
  // the query and weight loads and the histogram clear below overlap them
  i32x4 buf0[T::NI], buf1[T::NI];
  float ksc0 = 0.0f, ksc1 = 0.0f;
  int base = k0 + kDecodeWaveKeys * wave;
  if (base < k1) load_step(buf0, ksc0, base);
  if (base + kDecodeBlockKeys < k1) load_step(buf1, ksc1, base + kDecodeBlockKeys);

  static_assert(kDecodeHistBins % (4 * 256) == 0, "histogram clear");
#pragma unroll
  for (int i = 0; i < kDecodeHistBins / (4 * 256); ++i) ((uint4*)hist)[threadIdx.x + 256 * i] = make_uint4(0u, 0u, 0u, 0u);

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
  // lane weights: heads 32*mb + 8*(r/4) + 4g + r%4, four consecutive heads
  // per 16-byte load when every row of w starts 16-byte aligned (w itself
  // 16-byte aligned and H % 4 == 0; w need only be 4-byte aligned)
  float wr[MB][16];
  const float qs = FP8 ? p.q_scale[row] : 1.0f;
  if ((p.H & 3) == 0 && ((uintptr_t)p.w & 15u) == 0u) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int head = 32 * mb + 8 * j + 4 * g;
        const float4 x = head < p.H ? *(const float4*)(p.w + row * p.H + head) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        wr[mb][4 * j] = x.x * qs;
        wr[mb][4 * j + 1] = x.y * qs;
        wr[mb][4 * j + 2] = x.z * qs;
        wr[mb][4 * j + 3] = x.w * qs;
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int head = 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
        wr[mb][r] = head < p.H ? p.w[row * p.H + head] * qs : 0.0f;
      }
  }
  __syncthreads();  // histogram cleared

  // one step: rows to LDS, refill the buffer with the step two ahead, MFMAs
  // on fragments read from LDS, epilogue
  auto step = [&](i32x4 (&buf)[T::NI], float& ksc, int base) {
#pragma unroll
    for (int i = 0; i < T::NI; ++i) *(i32x4*)(lt + (T::RPI * i + lr) * T::RS + 16 * lc) = buf[i];
    const float ksc_cur = ksc;
    const int ahead = base + 2 * kDecodeBlockKeys;
    if (ahead < k1) load_step(buf, ksc, ahead);
    wave_sync();
    // B fragment: key base + i32, dims g*(D/2) + (8 bf16 | 32 fp8)*ks ..
    const unsigned char* fr = lt + i32 * T::RS + (FP8 ? g * (D / 2) : g * D);
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Frag kb;
      if constexpr (FP8) {
        const i32x4 lo = *(const i32x4*)(fr + 32 * ks), hi = *(const i32x4*)(fr + 32 * ks + 16);
        kb = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        kb = *(const bf16x8*)(fr + 16 * ks);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (FP8)
          acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][ks], kb, acc[mb], 0, 0, 0, 127, 0, 127);
        else
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
      }
    }
    // lane holds heads 32*mb + 8(r/4) + 4g + (r%4) of key base + i32
    float part = 0.0f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        part = __builtin_fmaf(wr[mb][r], __int_as_float(max(__float_as_int(acc[mb][r]), 0)), part);
    float score = part + __shfl_xor(part, 32, 64);
    if constexpr (FP8) score *= ksc_cur;
    const int key = base + i32;
    if (g == 0 && key < k1) {
      const uint32_t u = score_key(score);
      keys_out[key] = u;
      if constexpr (DUMP) p.dump[row * (size_t)p.n_k + key] = canon_zero(score);
      atomicAdd(&hist[u >> (32 - kDecodeHistBits)], 1u);
    }
  };

  for (; base < k1; base += 2 * kDecodeBlockKeys) {
    step(buf0, ksc0, base);
    if (base + kDecodeBlockKeys >= k1) break;
    step(buf1, ksc1, base + kDecodeBlockKeys);
  }
  __syncthreads();
  uint32_t* gh = p.dec_hist + (size_t)b * kDecodeHistRow + (blockIdx.x % kDecodeHistCopies) * kDecodeHistStride;
  for (int i = threadIdx.x; i < kDecodeHistBins; i += 256) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
  // coarse bins (64 fine bins each): thread t sums 16 fine bins, four threads
  // make one coarse bin
  static_assert(kDecodeHistBins == 256 * 16 && kDecodeCoarseBins * 64 == kDecodeHistBins, "histogram layout");
  uint32_t cs = 0u;
#pragma unroll
  for (int j = 0; j < 16; ++j) cs += hist[16 * threadIdx.x + j];
  cs += __shfl_xor(cs, 1, 64);
  cs += __shfl_xor(cs, 2, 64);
  if ((threadIdx.x & 3) == 0 && cs) atomicAdd(&gh[kDecodeHistBins + (threadIdx.x >> 2)], cs);
}

// Threshold bin of a request's histogram gh (its copies, each fine bins then
// coarse bins) by one wave: the largest T with count(bins >= T) >= k_eff,
// found in the coarse bins first and then among the 64 fine bins of the
// coarse bin found.
__device__ uint32_t sum_copies(const uint32_t* __restrict__ gh, int i) {
  uint32_t v[kDecodeHistCopies];
#pragma unroll
  for (int c = 0; c < kDecodeHistCopies; ++c) v[c] = gh[c * kDecodeHistStride + i];
  uint32_t s = 0u;
#pragma unroll
  for (int c = 0; c < kDecodeHistCopies; ++c) s += v[c];
  return s;
}
__device__ int wave_threshold_bin(const uint32_t* __restrict__ gh, int k_eff) {
  const int lane = lane_id();
  const uint32_t c = sum_copies(gh, kDecodeHistBins + kDecodeCoarseBins - 1 - lane);  // lane 0: top coarse bin
  const uint32_t ci = wave_incl_scan(c);
  const int L = uniform_i(__builtin_ctzll(ballot(ci >= (uint32_t)k_eff)));
  const uint32_t above = __shfl(ci - c, L, 64);  // keys in coarse bins above it
  const int cb = kDecodeCoarseBins - 1 - L;
  const uint32_t f = sum_copies(gh, 64 * cb + 63 - lane);
  const uint32_t fi = wave_incl_scan(f) + above;
  const int L2 = uniform_i(__builtin_ctzll(ballot(fi >= (uint32_t)k_eff)));
  return 64 * cb + 63 - L2;
}

// Appends every key whose top bits reach the threshold bin to the request's
// candidate list, in no particular order (the count may exceed C: the
// finalize kernel then takes the exact full-row select). One atomic per block
// reserves the block's slots.
__global__ __launch_bounds__(256) void decode_collect_kernel(IndexerParams p) {
  args_now(p.kv.seq_lens, p.pos_offset, p.n_k, p.topk, p.dec_hist, p.dec_keys, p.cand_cnt, p.cand_key, p.cand_idx, p.C,
           p.cnt_stride);
  __shared__ int scratch[17];
  __shared__ int sh_base;
  const int b = blockIdx.y;
  const int n_valid = decode_len(p.kv, b, p.pos_offset, p.n_k);
  if ((int)blockIdx.x * kDecodeCollectKeys >= n_valid) return;  // uniform: no keys here (or none at all)
  __shared__ int sh_tbin;
  if (threadIdx.x < kWave) {
    const int k_eff = min(p.topk, n_valid);
    const int tb = wave_threshold_bin(p.dec_hist + (size_t)b * kDecodeHistRow, k_eff);
    if (threadIdx.x == 0) sh_tbin = tb;
  }
  __syncthreads();
  const uint32_t tbin = (uint32_t)sh_tbin;
  const int beg = blockIdx.x * kDecodeCollectKeys, end = min(beg + kDecodeCollectKeys, n_valid);
  const uint32_t* keys = p.dec_keys + (size_t)b * decode_key_stride(p.n_k);
  constexpr int U = kDecodeCollectKeys / 256;
  static_assert(U == 16, "four 16-byte loads per thread");
  // thread t takes the U consecutive keys beg + U*t .. with four 16-byte
  // loads (rows are 256-byte aligned and padded to 64 keys, so a load that
  // starts before `end` stays inside the row)
  uint32_t u[U];
  {
    const int i0 = beg + U * (int)threadIdx.x;
    const uint4* src = (const uint4*)(keys + i0);
#pragma unroll
    for (int q = 0; q < U / 4; ++q) {
      const uint4 v = i0 < end ? src[q] : make_uint4(0u, 0u, 0u, 0u);
      u[4 * q] = v.x;
      u[4 * q + 1] = v.y;
      u[4 * q + 2] = v.z;
      u[4 * q + 3] = v.w;
    }
  }
  int n = 0;
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int i = beg + U * (int)threadIdx.x + j;
    n += (i < end && (u[j] >> (32 - kDecodeHistBits)) >= tbin) ? 1 : 0;
  }
  int total;
  int pos = block_excl_scan(n, scratch, &total);
  if (total == 0) return;
  if (threadIdx.x == 0) sh_base = atomicAdd(&p.cand_cnt[(size_t)b * p.cnt_stride], total);
  __syncthreads();
  pos += sh_base;
  uint32_t* ck = p.cand_key + (size_t)b * p.C;
  int32_t* ci = p.cand_idx + (size_t)b * p.C;
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int i = beg + U * (int)threadIdx.x + j;
    if (i < end && (u[j] >> (32 - kDecodeHistBits)) >= tbin) {
      if (pos < p.C) {
        ck[pos] = u[j];
        ci[pos] = i;
      }
      ++pos;
    }
  }
}

// Score blocks of a decode call: the planned list for ragged lengths, else
// (blocks per request, B) with about kDecodeTargetBlocks blocks in all, at
// least one block step each.
static dim3 decode_score_grid(const IndexerParams& p) {
  if (p.kv.seq_lens) return dim3(p.B + kDecodeTargetBlocks, 1);
  const int kend = std::min(p.pos_offset + 1, p.n_k);
  const int steps = (kend + kDecodeBlockKeys - 1) / kDecodeBlockKeys;
  const int nb = std::max(1, std::min(kDecodeTargetBlocks / p.B, steps));
  return dim3(nb, p.B);
}

template <int D, int MB, bool FP8>
static void launch_decode_scores_t(const IndexerParams& p, hipStream_t s) {
  const dim3 grid = decode_score_grid(p);
  if (p.dump)
    hipLaunchKernelGGL((indexer_decode_kernel<D, MB, FP8, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((indexer_decode_kernel<D, MB, FP8, false>), grid, dim3(256), 0, s, p);
}

hipError_t launch_indexer_decode(const IndexerParams& p, hipStream_t s) {
  // zero the histograms and counters (a kernel, not a memset node), and plan
  // ragged score blocks; a later F layer of a stack finds them zero (the
  // finalize kernel clears its request's row) and the plan built
  if (!p.skip_prepare) {
    const size_t nz = (size_t)p.B * kDecodeHistRow;
    hipLaunchKernelGGL(decode_prepare_kernel, dim3((unsigned)std::min<size_t>((nz + 255) / 256, 1024)), dim3(256), 0,
                       s, p, nz, p.B + kDecodeTargetBlocks);
  }
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
  const int n_max = p.kv.seq_lens ? p.n_k : std::min(p.pos_offset + 1, p.n_k);
  const int ncb = (n_max + kDecodeCollectKeys - 1) / kDecodeCollectKeys;
  hipLaunchKernelGGL(decode_collect_kernel, dim3(ncb, p.B), dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_topk_finalize(p, p.B, s);
  if (e != hipSuccess) return e;
  return record_phase(p.ev, 2, s);
}

}  // namespace dsa
