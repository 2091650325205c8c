// Sparse attention over the indexer's selected tokens: for query t, head h,
//   O[t,h] = softmax_r(scale * q[t,h] . K[idx[t,r]]) . V[idx[t,r]]
// over the valid entries r (0 <= idx <= pos(t), idx < n_k; -1 padding and any
// other out-of-range entry is skipped). One KV head is shared by all query
// heads, so each selected K/V row is gathered once per query and reused by
// every head.
//
// Mapping (gfx950, wave64): one wave per (query, split). The query's heads
// (padded to 16) are the M dimension of v_mfma_f32_16x16x32_bf16; each chunk
// of 32 selected keys gives two 16-key N blocks whose K rows are gathered
// straight from memory into B-fragments (a lane reads 16 contiguous bytes of
// one row per k-step). Online softmax runs in fp32 with exp2 (scale folded
// with log2 e). The P.V product runs on the VALU: each lane owns two
// contiguous output dims for every head, the wave gathers one V row per
// instruction (fully coalesced), and P is handed over through 2 KB of LDS
// per wave. Decode (one query per request) splits the index list over many
// waves and merges the partial (max, sum, O) triples in a second kernel.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kAttnWaves = 4;
constexpr int kAttnChunk = 32;

template <int D, bool SPLIT>
__global__ __launch_bounds__(kAttnWaves * kWave) void sparse_attn_kernel(AttnParams p) {
  constexpr int KS = D / 32;       // 16x16x32 k-steps over head_dim
  constexpr int RG = 128 / D;      // V rows per gather instruction (D=128: 1, D=64: 2)
  constexpr int DPL = 2;           // output dims per lane
  __shared__ __attribute__((aligned(16))) float lds_p[kAttnWaves][kAttnChunk][16];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int rows = p.B * p.n_q;
  const int row = blockIdx.x * kAttnWaves + wave;
  if (row >= rows) return;  // no workgroup barriers below
  const int b = row / p.n_q;
  const int t = row - b * p.n_q;
  const int pos = p.pos_offset + t;
  const int split = blockIdx.y;
  const int per = ((p.topk + p.nsplit - 1) / p.nsplit + kAttnChunk - 1) / kAttnChunk * kAttnChunk;
  const int e0 = split * per;
  const int e1 = min(e0 + per, p.topk);
  const int i16 = lane & 15, g = lane >> 4;
  const float sl2 = p.scale * 1.4426950408889634f;

  // Q fragments: head i16, dims g*(D/4) + 8*ks .. +7
  bf16x8 qa[KS];
  {
    const __bf16* qrow = (const __bf16*)p.q + ((size_t)row * p.H + i16) * D + g * (D / 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = {};
      if (i16 < p.H) v = *(const bf16x8*)(qrow + 8 * ks);
      qa[ks] = v;
    }
  }
  const __bf16* kb = (const __bf16*)p.k + (size_t)b * p.n_k * D;
  const __bf16* vb = (const __bf16*)p.v + (size_t)b * p.n_k * D;
  const int32_t* irow = p.idx + (size_t)row * p.topk;
  const int rg = (RG == 1) ? 0 : (lane >> 5);
  const int d0 = DPL * (RG == 1 ? lane : (lane & 31));

  float o[16][DPL];
#pragma unroll
  for (int h = 0; h < 16; ++h)
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[h][c] = 0.0f;
  float m[4], l[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -__builtin_inff();
    l[r] = 0.0f;
  }
  float (*P)[16] = lds_p[wave];

  for (int c0 = e0; c0 < e1; c0 += kAttnChunk) {
    const int e = c0 + (lane & 31);
    const int raw = e < e1 ? irow[e] : -1;
    const bool valid = raw >= 0 && raw <= pos && raw < p.n_k;
    const int key = valid ? raw : 0;
    float sv[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int kj = __shfl(key, 16 * nb + i16, 64);
      const int vj = __shfl(valid ? 1 : 0, 16 * nb + i16, 64);
      const __bf16* krow = kb + (size_t)kj * D + g * (D / 4);
      f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(krow + 8 * ks);
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kf, s, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[nb][r] = vj ? s[r] * sl2 : -__builtin_inff();
    }
    // online softmax; lane holds heads 4g + r of key 16*nb + i16
    float corr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mx = wave_max16(fmaxf(sv[0][r], sv[1][r]));
      const float mn = fmaxf(m[r], mx);
      const bool none = mn == -__builtin_inff();
      corr[r] = none ? 1.0f : exp2f(m[r] - mn);
      const float p0 = none ? 0.0f : exp2f(sv[0][r] - mn);
      const float p1 = none ? 0.0f : exp2f(sv[1][r] - mn);
      l[r] = l[r] * corr[r] + p0 + p1;
      m[r] = mn;
      P[i16][4 * g + r] = p0;
      P[16 + i16][4 * g + r] = p1;
    }
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      const float ch = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr[h & 3]), 16 * (h >> 2)));
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[h][c] *= ch;
    }
    wave_sync();
    // P.V on the VALU: one gathered V row per step
#pragma unroll 8
    for (int kq = 0; kq < kAttnChunk / RG; ++kq) {
      const int kk = kq * RG + rg;
      const int vk = __shfl(key, kk, 64);
      const uint32_t pair = *(const uint32_t*)(vb + (size_t)vk * D + d0);
      const float v0 = __uint_as_float(pair << 16);
      const float v1 = __uint_as_float(pair & 0xffff0000u);
      const f32x4* prow = (const f32x4*)P[kk];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 pp = prow[q4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[4 * q4 + j][0] = __builtin_fmaf(pp[j], v0, o[4 * q4 + j][0]);
          o[4 * q4 + j][1] = __builtin_fmaf(pp[j], v1, o[4 * q4 + j][1]);
        }
      }
    }
    wave_sync();
  }
  // reduce the per-lane partial sums over the 16 keys of each lane group
#pragma unroll
  for (int r = 0; r < 4; ++r) l[r] = wave_sum16(l[r]);
  if (RG == 2) {
#pragma unroll
    for (int h = 0; h < 16; ++h)
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[h][c] += __shfl_xor(o[h][c], 32, 64);
  }
  const bool writer = (RG == 1) || lane < 32;
  for (int h = 0; h < p.H; ++h) {
    const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m[h & 3]), 16 * (h >> 2)));
    const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l[h & 3]), 16 * (h >> 2)));
    if constexpr (SPLIT) {
      float* dst = p.part + (((size_t)row * p.nsplit + split) * p.H + h) * (D + 2);
      if (writer) {
        dst[d0] = o[h][0];
        dst[d0 + 1] = o[h][1];
      }
      if (lane == 0) {
        dst[D] = mh;
        dst[D + 1] = lh;
      }
    } else {
      const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
      if (writer) {
        __bf16* dst = (__bf16*)p.out + ((size_t)row * p.H + h) * D + d0;
        dst[0] = (__bf16)(o[h][0] * inv);
        dst[1] = (__bf16)(o[h][1] * inv);
      }
      if (p.lse && lane == 0)
        p.lse[(size_t)row * p.H + h] = lh > 0.0f ? (mh + __log2f(lh)) * 0.6931471805599453f
                                                 : -__builtin_inff();
    }
  }
}

// Merges the split partials: M = max_s m_s, L = sum_s l_s 2^(m_s - M),
// O = sum_s o_s 2^(m_s - M) / L  (m in log2 units).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  const int row = blockIdx.x;
  const int ns = p.nsplit;
  for (int e = threadIdx.x; e < p.H * D; e += blockDim.x) {
    const int h = e / D, d = e - h * D;
    const float* base = p.part + ((size_t)row * ns * p.H + h) * (D + 2);
    const size_t sstride = (size_t)p.H * (D + 2);
    float M = -__builtin_inff();
    for (int s = 0; s < ns; ++s) M = fmaxf(M, base[s * sstride + D]);
    float L = 0.0f, O = 0.0f;
    if (M != -__builtin_inff()) {
      for (int s = 0; s < ns; ++s) {
        const float ms = base[s * sstride + D];
        const float f = ms == -__builtin_inff() ? 0.0f : exp2f(ms - M);
        L += base[s * sstride + D + 1] * f;
        O += base[s * sstride + d] * f;
      }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    ((__bf16*)p.out)[((size_t)row * p.H + h) * D + d] = (__bf16)(O * inv);
    if (p.lse && d == 0)
      p.lse[(size_t)row * p.H + h] = L > 0.0f ? (M + __log2f(L)) * 0.6931471805599453f : -__builtin_inff();
  }
}

template <int D>
static hipError_t launch_attn_t(const AttnParams& p, hipStream_t s) {
  const int rows = p.B * p.n_q;
  const dim3 grid((rows + kAttnWaves - 1) / kAttnWaves, p.nsplit);
  if (p.nsplit > 1) {
    hipLaunchKernelGGL((sparse_attn_kernel<D, true>), grid, dim3(kAttnWaves * kWave), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3(rows), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((sparse_attn_kernel<D, false>), grid, dim3(kAttnWaves * kWave), 0, s, p);
  }
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
