// Device-side helpers shared by the libdsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Order-preserving 32-bit key of an fp32 score: a > b  <=>  key(a) > key(b),
// with -0.0 mapped to the key of +0.0. Finite scores map to keys >= 0x00800000,
// so the key 0 lies below every score.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// score_key of a score that is not -0.0: a negative score flips every bit, a
// positive one only the sign bit.
__device__ __forceinline__ uint32_t score_key_nz(float s) {
  const uint32_t b = __float_as_uint(s);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(b);
}

// -0.0 -> +0.0 (bit-level, immune to fast-math folding).
__device__ __forceinline__ float canon_zero(float s) {
  uint32_t b = __float_as_uint(s);
  return __uint_as_float(b == 0x80000000u ? 0u : b);
}

// (the range lets the compiler narrow lane arithmetic and fold lane guards)
__device__ __forceinline__ int lane_id() {
  const int l = __lane_id();
  __builtin_assume(l >= 0 && l < kWave);
  return l;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Kernel arguments sit in memory the host has just written, so each batch of
// argument loads that waits for an earlier one (a load behind a branch on
// another argument, the grid size read once the block's range is needed)
// costs one more trip to HBM, about a microsecond, before a short kernel
// issues its first data load. The short decode kernels name every argument
// they use at entry, which puts all of those loads in one batch.
__device__ __forceinline__ void arg_now(const void* v) { asm volatile("" ::"s"(v)); }
__device__ __forceinline__ void arg_now(int v) { asm volatile("" ::"s"(v)); }
__device__ __forceinline__ void arg_now(unsigned v) { asm volatile("" ::"s"(v)); }
__device__ __forceinline__ void arg_now(float v) { asm volatile("" ::"s"(v)); }
template <typename... T>
__device__ __forceinline__ void args_now(const T&... v) {
  (arg_now(v), ...);
}
__device__ __forceinline__ uint32_t uniform_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Orders this wave's earlier LDS and global accesses before its later ones, for
// all lanes of the wave (cross-lane hand-over through memory inside one wave).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ float wave_max16(float v) {
  // max over the 16 lanes of each aligned group of 16
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

__device__ __forceinline__ float wave_sum16(float v) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}

}  // namespace dsa
