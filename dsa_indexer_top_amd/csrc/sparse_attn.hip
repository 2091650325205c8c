// Sparse attention over the indexer's selected tokens: for query t, head h,
//   O[t,h] = softmax_r(scale * q[t,h] . K[idx[t,r]]) . V[idx[t,r]]
// over the valid entries r (0 <= idx <= pos(t), idx < n_k; -1 padding and any
// other out-of-range entry is skipped). One KV head is shared by all query
// heads, so each selected K/V row is gathered once per query and reused by
// every head.
//
// Mapping (gfx950, wave64): one wave per (query, split); the wave walks its
// slice of the index list in chunks of 32 entries. Both products run on
// v_mfma_f32_16x16x32_bf16 with the query's heads (padded to 16) as the
// 16-wide N dimension:
//   S^T[key, head] = K_sel . Q^T   A = gathered K rows (a lane reads 16
//                                  contiguous bytes of one row per k-step),
//                                  B = Q^T (kept in registers);
//   O^T[dim, head] += V_sel^T . P^T
// The S^T accumulator leaves every lane with one head and 8 keys, which is
// exactly the B operand P^T of the second product (its k-slots are those 8
// keys), so the probabilities never leave registers and each lane's softmax
// state (running max, partial sum) is one scalar for its head. The A operand
// V^T needs 8 keys of one dim per lane: the chunk's 32 V rows are gathered
// with 16-byte coalesced loads, keys j and j + 16 are interleaved per dim
// with v_perm (one dword = that dim of both keys) and staged in LDS as 16
// "pair rows", so each A-operand dword is a single 32-bit LDS read (rows
// padded so the four lane groups of a read hit disjoint banks). Online
// softmax in fp32 with exp2 (scale folded with log2 e); P is rounded to bf16
// for the second product.
// Few rows (decode, short prefill chunks) split each row's list over several
// waves (split-K) so that about 2048 waves share the call. Up to 4 splits
// each wave writes its (O, max, sum) partial; from 8 splits on, the splits
// of a workgroup are merged in LDS first: at 8 splits one workgroup of 8
// waves covers the row and writes the output, from 16 splits on workgroups
// of 4 waves each write one partial (at most 16 per row). A second kernel
// merges a row's partials by the log-sum-exp rule.
// A wave with more than one chunk gathers the next chunk's K rows while it
// computes the current one (its V rows are requested at its start, ahead of
// its S product); a wave with one chunk gathers K and V together.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kAttnWaves = 4;  // waves per workgroup when every wave is on its own
constexpr int kAttnChunk = 32;

// Launch forms: one wave per row writing the output; one wave per split
// writing a partial; workgroups of split waves that merge in LDS and write
// the output (one 8-wave workgroup per row) or one partial each (4-wave
// workgroups).
enum AttnMode { kAttnDirect = 0, kAttnSplit = 1, kAttnGroup = 2 };

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct AttnShape {
  static constexpr int KS = D / 32;           // k-steps of S^T over head_dim
  static constexpr int DB = D / 16;           // 16-dim blocks of O^T
  static constexpr int LPR = D / 8;           // lanes per V row (16 B each)
  static constexpr int RPI = kWave / LPR;     // V rows per load instruction
  static constexpr int VL = kAttnChunk / RPI; // V load instructions per chunk
  static constexpr int PSTRIDE = 4 * D + 64;  // LDS bytes per pair row (D dwords + pad)
};

// LDS pair row of the key pair (j, j + 16), j < 16: pair 4g + w sits in row
// 4w + g, so the four lane groups of a read (pairs 4 apart) touch consecutive
// rows, which a stride of 4D + 64 bytes places 16 banks apart.
__device__ __forceinline__ int prow(int j) { return (j & 3) * 4 + (j >> 2); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int MODE, int WAVES, bool PIPE>
__device__ __forceinline__ void sparse_attn_body(const AttnParams& p) {
  using S = AttnShape<D>;
  static_assert((S::PSTRIDE / 4) % 64 == 16, "lane groups of a read must not share banks");
  __shared__ __attribute__((aligned(16))) unsigned char lds_v[WAVES][16 * S::PSTRIDE];
  args_now(p.nsplit, p.B, p.n_q, p.n_k, p.pos_offset, p.topk, p.H, p.scale, p.q, p.k, p.v, p.idx, p.part, p.out, p.lse,
           p.kv.seq_lens, p.kv.block_table);
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  __builtin_assume(wave >= 0 && wave < WAVES);
  const int ns = p.nsplit;
  int row, split, wid;  // wid: this wave's (or workgroup's) partial
  if constexpr (MODE == kAttnGroup) {
    const int groups = ns / WAVES;  // workgroups per row
    row = blockIdx.x / groups;
    wid = blockIdx.x;
    split = (blockIdx.x - row * groups) * WAVES + wave;
  } else {
    wid = blockIdx.x * WAVES + wave;
    if (wid >= p.B * p.n_q * ns) return;  // no workgroup barriers in these forms
    row = wid / ns;
    split = wid - row * ns;
  }
  const int b = row / p.n_q;
  const int t = row - b * p.n_q;
  const bool paged = p.kv.block_table != nullptr;  // decode over page pools (n_q == 1)
  const int pos = p.kv.seq_lens ? decode_len(p.kv, b, 0, p.n_k) - 1 : p.pos_offset + t;
  const int per = ((p.topk + ns - 1) / ns + kAttnChunk - 1) / kAttnChunk * kAttnChunk;
  const int e0 = split * per;
  const int e1 = min(e0 + per, p.topk);
  const int i16 = lane & 15, g = lane >> 4;
  const float sl2 = p.scale * 1.4426950408889634f;

  // Q^T as the B operand: column = head i16, k-slots = dims g*(D/4) + 8*ks .. +7
  bf16x8 qb[S::KS];
  {
    const __bf16* qrow = (const __bf16*)p.q + ((size_t)row * p.H + i16) * D + g * (D / 4);
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      bf16x8 v = {};
      if (i16 < p.H) v = *(const bf16x8*)(qrow + 8 * ks);
      qb[ks] = v;
    }
  }
  const unsigned char* kb = (const unsigned char*)p.k + (paged ? 0 : (size_t)b * p.n_k * D * 2);
  const unsigned char* vb = (const unsigned char*)p.v + (paged ? 0 : (size_t)b * p.n_k * D * 2);
  const int32_t* irow = p.idx + (size_t)row * p.topk;
  unsigned char* vl = lds_v[wave];
  const int vr = lane / S::LPR, vc = lane % S::LPR;  // V load: row in group, 16-byte column

  f32x4 o[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) o[db] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float m = -__builtin_inff(), l = 0.0f;

  struct Chunk {
    bf16x8 kf[2][S::KS];
    i32x4 vv[S::VL];  // !PIPE: gathered with K
    uint32_t vmask;
    int key;
  };
  // index entries of the chunk at c (lanes l and l + 32: entry c + l % 32)
  auto load_idx = [&](int c) -> int {
    const int e = c + (lane & 31);
    return e < e1 ? irow[e] : -1;
  };
  // a chunk's gathers: K rows as A fragments, V rows into registers
  auto gather = [&](Chunk& ch, int raw) {
    const bool valid = raw >= 0 && raw <= pos && raw < p.n_k;
    // K/V row of this entry: the token itself, or its pool row under paging
    // (an invalid entry reads row 0 of the request, or of the pool; its weight is 0)
    const int key = !valid ? 0 : (paged ? (int)paged_row(p.kv, b, raw) : raw);
    ch.vmask = (uint32_t)ballot(valid);  // bit j: entry j of the chunk is valid
    ch.key = key;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int kj = __shfl(key, 16 * nb + i16, 64);
      const unsigned char* krow = kb + (size_t)kj * (D * 2) + g * (D / 2);
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) ch.kf[nb][ks] = *(const bf16x8*)(krow + 16 * ks);
    }
    if constexpr (!PIPE) {
#pragma unroll
      for (int i = 0; i < S::VL; ++i) {
        const int vj = __shfl(key, S::RPI * i + vr, 64);
        ch.vv[i] = *(const i32x4*)(vb + (size_t)vj * (D * 2) + 16 * vc);
      }
    }
  };
  auto compute = [&](const Chunk& ch) {
    const uint32_t vmask = ch.vmask;
    i32x4 vv[S::VL];
#pragma unroll
    for (int i = 0; i < S::VL; ++i) {
      if constexpr (PIPE) {
        const int vj = __shfl(ch.key, S::RPI * i + vr, 64);
        vv[i] = *(const i32x4*)(vb + (size_t)vj * (D * 2) + 16 * vc);
      } else {
        vv[i] = ch.vv[i];
      }
    }
    // S^T = K . Q^T: lane holds head i16, keys 16*nb + 4*g + r
    f32x4 s[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      s[nb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) s[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.kf[nb][ks], qb[ks], s[nb], 0, 0, 0);
    }

    // stage V as pair rows: load i holds keys RPI*i + vr, load i + VL/2 the
    // keys 16 later; one output dword = (key j, key j + 16) of one dim.
    // (The previous chunk's reads of this wave's buffer are complete: LDS
    // operations of one wave execute in order.)
    wave_sync();
#pragma unroll
    for (int i = 0; i < S::VL / 2; ++i) {
      const i32x4 lo = vv[i], hi = vv[i + S::VL / 2];
      i32x4 x, y;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        x[2 * c] = __builtin_amdgcn_perm(hi[c], lo[c], 0x05040100u);
        x[2 * c + 1] = __builtin_amdgcn_perm(hi[c], lo[c], 0x07060302u);
        y[2 * c] = __builtin_amdgcn_perm(hi[2 + c], lo[2 + c], 0x05040100u);
        y[2 * c + 1] = __builtin_amdgcn_perm(hi[2 + c], lo[2 + c], 0x07060302u);
      }
      unsigned char* dst = vl + prow(S::RPI * i + vr) * S::PSTRIDE + 32 * vc;
      *(i32x4*)dst = x;
      *(i32x4*)(dst + 16) = y;
    }

    // online softmax for head i16 (replicated over the four lane groups)
    float sv[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * nb + 4 * g + r;
        const float x = ((vmask >> j) & 1u) ? s[nb][r] * sl2 : -__builtin_inff();
        sv[4 * nb + r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const bool none = mn == -__builtin_inff();
    const float corr = none ? 1.0f : exp2_fast(m - mn);
    // P^T as the B operand; k-slot (g, 2w) is key 4g + w, (g, 2w + 1) key 16 + 4g + w
    bf16x8 pb;
    float psum = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = none ? 0.0f : exp2_fast(sv[w] - mn);
      const float p1 = none ? 0.0f : exp2_fast(sv[4 + w] - mn);
      psum += p0 + p1;
      pb[2 * w] = (__bf16)p0;
      pb[2 * w + 1] = (__bf16)p1;
    }
    l = l * corr + psum;
    m = mn;
#pragma unroll
    for (int db = 0; db < S::DB; ++db) o[db] *= corr;
    wave_sync();

    // O^T += V^T . P^T with the same k-slot order: dword w of the A operand is
    // the pair row of pair 4g + w at dim 16*db + i16
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      i32x4 a;
#pragma unroll
      for (int w = 0; w < 4; ++w) a[w] = *(const int*)(vl + prow(4 * g + w) * S::PSTRIDE + 4 * (16 * db + i16));
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, o[db], 0, 0, 0);
    }
  };

  if constexpr (PIPE) {
    // the next chunk's K rows are gathered while this chunk is computed (its
    // V rows are requested at its start, ahead of its S product); each index
    // load is issued before the gathers it does not feed
    Chunk ca, cb;
    int ra = load_idx(e0);
    int rb = load_idx(e0 + kAttnChunk);
    if (e0 < e1) gather(ca, ra);
    for (int c0 = e0; c0 < e1; c0 += 2 * kAttnChunk) {
      ra = load_idx(c0 + 2 * kAttnChunk);
      const bool has_b = c0 + kAttnChunk < e1;
      if (has_b) gather(cb, rb);
      compute(ca);
      if (!has_b) break;
      rb = load_idx(c0 + 3 * kAttnChunk);
      if (c0 + 2 * kAttnChunk < e1) gather(ca, ra);
      compute(cb);
    }
  } else {
    // one chunk at a time, K and V gathered together (waves with one chunk)
    Chunk ca;
    int raw_next = load_idx(e0);
    for (int c0 = e0; c0 < e1; c0 += kAttnChunk) {
      const int raw = raw_next;
      raw_next = load_idx(c0 + kAttnChunk);
      gather(ca, raw);
      compute(ca);
    }
  }
  // the four lane groups summed different keys of the same head
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if constexpr (MODE == kAttnGroup) {
    // each wave's (O, max, sum) into its own V buffer (its last reads of it
    // are done: a wave's LDS operations execute in order) as O [16][D], the
    // 16 maxima, the 16 sums; then the workgroup merges its WAVES splits per
    // (head, dim) by the log-sum-exp rule
    static_assert((16 * D + 32) * 4 <= 16 * S::PSTRIDE, "partial fits the V buffer");
    float* mine = (float*)vl;
#pragma unroll
    for (int db = 0; db < S::DB; ++db) *(f32x4*)(mine + i16 * D + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      mine[16 * D + i16] = m;
      mine[16 * D + 16 + i16] = l;
    }
    __syncthreads();
    constexpr int DPT = 16 * D / (WAVES * kWave);  // dims per thread
    constexpr int TPH = D / DPT;                   // threads per head
    static_assert(DPT % 2 == 0 && DPT * WAVES * kWave == 16 * D, "merge layout");
    const int h = threadIdx.x / TPH, d0 = (threadIdx.x % TPH) * DPT;
    if (h >= p.H) return;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, ((const float*)lds_v[w])[16 * D + h]);
    float L = 0.0f, acc[DPT];
#pragma unroll
    for (int c = 0; c < DPT; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float* pw = (const float*)lds_v[w];
      const float mw = pw[16 * D + h];
      const float f = mw == -__builtin_inff() ? 0.0f : exp2_fast(mw - M);
      L = __builtin_fmaf(pw[16 * D + 16 + h], f, L);
#pragma unroll
      for (int c = 0; c < DPT; c += 2) {
        const f32x2 x = *(const f32x2*)(pw + h * D + d0 + c);
        acc[c] = __builtin_fmaf(f, x[0], acc[c]);
        acc[c + 1] = __builtin_fmaf(f, x[1], acc[c + 1]);
      }
    }
    if (ns > WAVES) {  // one partial per workgroup, merged by attn_combine_kernel
      float* dst = p.part + ((size_t)wid * p.H + h) * kAttnPartStride<D>;
#pragma unroll
      for (int c = 0; c < DPT; c += 2) *(f32x2*)(dst + d0 + c) = (f32x2){acc[c], acc[c + 1]};
      if (d0 == 0) {
        dst[D] = M;
        dst[D + 1] = L;
      }
      return;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    __bf16* dst = (__bf16*)p.out + ((size_t)row * p.H + h) * D + d0;
#pragma unroll
    for (int c = 0; c < DPT; ++c) dst[c] = (__bf16)(acc[c] * inv);
    if (p.lse && d0 == 0)
      p.lse[(size_t)row * p.H + h] = L > 0.0f ? (M + __log2f(L)) * 0.6931471805599453f : -__builtin_inff();
    return;
  }
  if (i16 >= p.H) return;
  // lane holds O[head i16][16*db + 4*g + r]
  if constexpr (MODE == kAttnSplit) {
    float* dst = p.part + ((size_t)wid * p.H + i16) * kAttnPartStride<D>;
#pragma unroll
    for (int db = 0; db < S::DB; ++db) *(f32x4*)(dst + 16 * db + 4 * g) = o[db];
    if (g == 0) {
      dst[D] = m;
      dst[D + 1] = l;
    }
  } else {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    __bf16* dst = (__bf16*)p.out + ((size_t)row * p.H + i16) * D + 4 * g;
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)(o[db][r] * inv);
      *(bf16x4*)(dst + 16 * db) = v;
    }
    if (p.lse && g == 0)
      p.lse[(size_t)row * p.H + i16] = l > 0.0f ? (m + __log2f(l)) * 0.6931471805599453f : -__builtin_inff();
  }
}

// Waves with one chunk keep the compiler's occupancy choice. With the next
// chunk's K fragments in flight, the D = 128 kernels need more than 128
// registers (VGPRs and AGPRs together), so they are held to two waves per SIMD
// (256), which they fit without spilling.
template <int D, int MODE, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void sparse_attn_kernel(AttnParams p) {
  sparse_attn_body<D, MODE, WAVES, false>(p);
}
template <int D, int MODE, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_pipe_kernel(
    AttnParams p) {
  sparse_attn_body<D, MODE, WAVES, true>(p);
}

// Merges the partials of one (query, head) per wave:
// M = max_s m_s, L = sum_s l_s 2^(m_s - M), O = sum_s o_s 2^(m_s - M) / L
// (m in log2 units; a partial with no valid entry has m = -inf, l = 0, o = 0).
template <int D, int NS>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  constexpr int DPL = D / kWave;  // output dims per lane
  args_now(p.H, p.nsplit, p.part, p.out, p.lse);
  const int lane = lane_id();
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int row = blockIdx.y;
  if (h >= p.H) return;
  const int ns = attn_nparts(p.nsplit);  // <= NS
  const size_t sstride = (size_t)p.H * kAttnPartStride<D>;
  const float* base = p.part + ((size_t)row * ns * p.H + h) * kAttnPartStride<D>;
  // every split's partial O first (independent of the weights), then m and l,
  // so all loads are in flight together
  const float* src = base + DPL * lane;
  float v[NS][DPL];
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int c = 0; c < DPL; ++c) v[j][c] = j < ns ? src[j * sstride + c] : 0.0f;
  const float ms = lane < ns ? base[lane * sstride + D] : -__builtin_inff();
  const float ls = lane < ns ? base[lane * sstride + D + 1] : 0.0f;
  float M = ms;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
  const float f = (ms == -__builtin_inff()) ? 0.0f : exp2_fast(ms - M);
  float L = ls * f;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) L += __shfl_xor(L, d, 64);
  float o[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) o[c] = 0.0f;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const float fs = j < ns ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j)) : 0.0f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[c] = __builtin_fmaf(fs, v[j][c], o[c]);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  __bf16* dst = (__bf16*)p.out + ((size_t)row * p.H + h) * D + DPL * lane;
#pragma unroll
  for (int c = 0; c < DPL; ++c) dst[c] = (__bf16)(o[c] * inv);
  if (p.lse && lane == 0)
    p.lse[(size_t)row * p.H + h] = L > 0.0f ? (M + __log2f(L)) * 0.6931471805599453f : -__builtin_inff();
}

template <int D, bool PIPE>
static void launch_attn_form(const AttnParams& p, hipStream_t s) {
  const int rows = p.B * p.n_q;
  const int ns = p.nsplit;
  const dim3 grid((unsigned)(((long)rows * ns + kAttnWaves - 1) / kAttnWaves));
  const dim3 ggrid((unsigned)(rows * (ns / attn_group_waves(ns))));
  if constexpr (PIPE) {
    if (ns > kAttnGroupSplits)
      hipLaunchKernelGGL((sparse_attn_pipe_kernel<D, kAttnGroup, 4>), ggrid, dim3(4 * kWave), 0, s, p);
    else if (ns == kAttnGroupSplits)
      hipLaunchKernelGGL((sparse_attn_pipe_kernel<D, kAttnGroup, kAttnGroupSplits>), ggrid,
                         dim3(kAttnGroupSplits * kWave), 0, s, p);
    else if (ns > 1)
      hipLaunchKernelGGL((sparse_attn_pipe_kernel<D, kAttnSplit, kAttnWaves>), grid, dim3(kAttnWaves * kWave), 0, s, p);
    else
      hipLaunchKernelGGL((sparse_attn_pipe_kernel<D, kAttnDirect, kAttnWaves>), grid, dim3(kAttnWaves * kWave), 0, s, p);
  } else {
    if (ns > kAttnGroupSplits)
      hipLaunchKernelGGL((sparse_attn_kernel<D, kAttnGroup, 4>), ggrid, dim3(4 * kWave), 0, s, p);
    else if (ns == kAttnGroupSplits)
      hipLaunchKernelGGL((sparse_attn_kernel<D, kAttnGroup, kAttnGroupSplits>), ggrid, dim3(kAttnGroupSplits * kWave),
                         0, s, p);
    else if (ns > 1)
      hipLaunchKernelGGL((sparse_attn_kernel<D, kAttnSplit, kAttnWaves>), grid, dim3(kAttnWaves * kWave), 0, s, p);
    else
      hipLaunchKernelGGL((sparse_attn_kernel<D, kAttnDirect, kAttnWaves>), grid, dim3(kAttnWaves * kWave), 0, s, p);
  }
}

template <int D>
static hipError_t launch_attn_t(const AttnParams& p, hipStream_t s) {
  const int rows = p.B * p.n_q;
  const int ns = p.nsplit;
  if (ns < 1 || ns > 64 || (ns >= kAttnGroupSplits && ns % attn_group_waves(ns)) || attn_nparts(ns) > kAttnMaxParts)
    return hipErrorInvalidValue;
  // chunks per wave (the kernel's split of the list): prefetch only with more than one
  const int per = ((p.topk + ns - 1) / ns + kAttnChunk - 1) / kAttnChunk;
  if (per > 1) launch_attn_form<D, true>(p, s);
  else launch_attn_form<D, false>(p, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || attn_nparts(ns) <= 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<D, kAttnMaxParts>), dim3((p.H + 3) / 4, rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnParams& p, hipStream_t s) {
  hipError_t e = record_phase(p.ev, 0, s);
  if (e != hipSuccess) return e;
  if (p.D == 64) e = launch_attn_t<64>(p, s);
  else if (p.D == 128) e = launch_attn_t<128>(p, s);
  else e = hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  return record_phase(p.ev, 1, s);
}

}  // namespace dsa
