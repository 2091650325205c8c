// Per-token fp8 quantisation of indexer inputs (bf16 -> OCP e4m3fn codes plus
// one fp32 scale per row):
//   scale = fl32(amax / 448) (1 for an all-zero row),
//   code  = e4m3fn(fl32(x / scale)), round to nearest, ties to the even
//           mantissa, magnitudes clamped to 448.
// One wave per row: amax is a wave max over the row, then every value is
// divided, clamped to +-448 (the largest finite e4m3fn magnitude) and
// converted by v_cvt_pk_fp8_f32 (OCP e4m3fn, round to nearest even on gfx950;
// the clamp keeps it away from its out-of-range results), 8 codes per lane.
//
// The division. The scale is one per row, so the row's reciprocal
// y = fl32(1 / s) is taken once (IEEE division) and each quotient by the
// correction of Markstein's theorem (Markstein, IBM J. Res. Dev. 34(1), 1990;
// Muller et al., Handbook of Floating-Point Arithmetic, the FMA-based
// division chapter): q = fl32(x y), e = fma(-q, s, x) (exact), q' = fma(e, y, q)
// is the correctly rounded x / s when nothing underflows. Three operations
// per value instead of the ~10 of a full IEEE division. Where the residual e
// underflows (tiny x and s), q' can differ from fl32(x / s) in its low bits;
// with s >= 2^-100 that happens only for quotients below 2^-13, under half
// the smallest e4m3fn magnitude (2^-10), so the code is a signed zero either
// way. The sign is restored from x, since a -0 input would otherwise come out
// +0. A standalone exhaustive check of every bf16 x against every bf16 row
// maximum amax with s >= 2^-100 (1.04e9 pairs, |x| <= amax) gave identical
// codes (largest deviating quotient 1.2e-4). Rows with a smaller scale
// divide exactly.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kQuantWaves = 4;

// Rows of up to kQuantRegCols values stay in registers (all of a lane's loads
// in flight at once, one pass over memory); longer rows take two passes.
constexpr int kQuantRegChunks = 16;
constexpr int kQuantRegCols = 8 * kWave * kQuantRegChunks;

// fl32(x / s) (x / s when `fast` is false), with y = fl32(1 / s); see above
__device__ __forceinline__ float quotient(float x, float s, float y, bool fast) {
  if (!fast) return x / s;
  const float q = x * y;
  const float e = __builtin_fmaf(-q, s, x);
  const float r = __builtin_fmaf(e, y, q);
  return __uint_as_float((__float_as_uint(r) & 0x7fffffffu) | (__float_as_uint(x) & 0x80000000u));
}

// the row's scale s, its reciprocal y and whether the fast quotient applies
struct RowScale {
  float s, y;
  bool fast;
};
__device__ __forceinline__ RowScale row_scale(float amax) {
  RowScale r;
  r.s = amax > 0.0f ? amax / 448.0f : 1.0f;  // IEEE binary32 division
  r.fast = r.s >= 0x1p-100f;
  r.y = r.fast ? 1.0f / r.s : 0.0f;
  return r;
}

// 8 codes: the hardware pair conversion (round to nearest even) after the
// clamp to +-448, so it never sees an out-of-range value
__device__ __forceinline__ uint2 encode8(const bf16x8& v, const RowScale& rs) {
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    y[j] = __builtin_fminf(__builtin_fmaxf(quotient((float)v[j], rs.s, rs.y, rs.fast), -448.0f), 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

__device__ __forceinline__ float wave_amax(float a) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) a = fmaxf(a, __shfl_xor(a, d, 64));
  return a;
}

__global__ __launch_bounds__(kQuantWaves * kWave) void quantize_fp8_rows_kernel(const __bf16* __restrict__ x,
                                                                                  int64_t rows, int cols,
                                                                                  uint8_t* __restrict__ out,
                                                                                  float* __restrict__ scale) {
  const int lane = lane_id();
  const int64_t r = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  if (r >= rows) return;
  const __bf16* xr = x + r * cols;
  uint8_t* orow = out + r * cols;
  if (cols <= kQuantRegCols) {
    bf16x8 v[kQuantRegChunks];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kQuantRegChunks; ++i) {
      const int c = 8 * lane + 8 * kWave * i;
      v[i] = c < cols ? *(const bf16x8*)(xr + c) : (bf16x8){};
    }
#pragma unroll
    for (int i = 0; i < kQuantRegChunks; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf((float)v[i][j]));
    amax = wave_amax(amax);
    const RowScale rs = row_scale(amax);
    if (lane == 0) scale[r] = rs.s;
#pragma unroll
    for (int i = 0; i < kQuantRegChunks; ++i) {
      const int c = 8 * lane + 8 * kWave * i;
      if (c < cols) *(uint2*)(orow + c) = encode8(v[i], rs);
    }
    return;
  }
  float amax = 0.0f;
  for (int c = 8 * lane; c < cols; c += 8 * kWave) {
    const bf16x8 v = *(const bf16x8*)(xr + c);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf((float)v[j]));
  }
  amax = wave_amax(amax);
  const RowScale rs = row_scale(amax);
  if (lane == 0) scale[r] = rs.s;
  for (int c = 8 * lane; c < cols; c += 8 * kWave) *(uint2*)(orow + c) = encode8(*(const bf16x8*)(xr + c), rs);
}

hipError_t launch_quantize_fp8_rows(const void* x, int64_t rows, int cols, void* out, float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows + kQuantWaves - 1) / kQuantWaves;
  hipLaunchKernelGGL(quantize_fp8_rows_kernel, dim3((unsigned)blocks), dim3(kQuantWaves * kWave), 0, s,
                     (const __bf16*)x, rows, cols, (uint8_t*)out, scale);
  return hipGetLastError();
}

}  // namespace dsa
