// Device-side helpers shared by the gfx950 kernels: bf16 packing, ordered
// float keys for exact top-k, wave reductions and MFMA fragment types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef uint16_t bf16_t;  // raw bf16 bits in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Round-to-nearest-even fp32 -> bf16 for a pair (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
// -0.0 is folded onto +0.0 so that the two compare equal, as floats do.
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave64 reductions through DPP/permute (results valid in every lane).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Number of set bits of a 64-bit ballot below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Exact integer budget rule: k = min(n, max(min_blocks, ceil(ratio_q16 * n / 2^16))).
__host__ __device__ __forceinline__ int budget_blocks(int n, int min_blocks, uint32_t ratio_q16) {
  long long want = ((long long)ratio_q16 * (long long)n + 65535ll) >> 16;
  if (want < min_blocks) want = min_blocks;
  return want < n ? int(want) : n;
}

}  // namespace sa
