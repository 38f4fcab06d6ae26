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
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

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

// Cross-lane moves that stay in the VALU (no LDS round trip):
//   dpp<CTRL>   data-parallel primitive move (quad_perm 0x00-0xFF,
//               row_mirror 0x140, row_half_mirror 0x141) inside 16-lane rows;
//   swap16/32   v_permlane16_swap / v_permlane32_swap with both operands equal:
//               the two results hold a value and its partner's (lane ^ 16 /
//               lane ^ 32), so combining them gives the pairwise reduction.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum / max over the 16 lanes of each row, result in every lane.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8-lane half
  x += dpp<0x140>(x);  // row_mirror: the other half of the row
  return x;
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}
// Sum over the 8 lanes of each half-row (lanes 8r .. 8r+7), result in every lane.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x;
}

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (lanes a shift or a row mask leaves out add 0).
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Unsigned min / max over the 64 lanes (every lane active), result in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
  x = min(x, dpp_u32<0xB1>(x));
  x = min(x, dpp_u32<0x4E>(x));
  x = min(x, dpp_u32<0x141>(x));
  x = min(x, dpp_u32<0x140>(x));
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = min(uint32_t(r[0]), uint32_t(r[1]));
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return min(uint32_t(r[0]), uint32_t(r[1]));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = max(x, dpp_u32<0xB1>(x));
  x = max(x, dpp_u32<0x4E>(x));
  x = max(x, dpp_u32<0x141>(x));
  x = max(x, dpp_u32<0x140>(x));
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(uint32_t(r[0]), uint32_t(r[1]));
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(uint32_t(r[0]), uint32_t(r[1]));
}

// Wave64 reductions, result valid in every lane.
__device__ __forceinline__ float wave_max(float x) { return max_xor32(max_xor16(row_max16(x))); }
__device__ __forceinline__ float wave_sum(float x) { return sum_xor32(sum_xor16(row_sum16(x))); }
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

__device__ __forceinline__ u32x4 lds16(const char* base, int off) { return *reinterpret_cast<const u32x4*>(base + off); }

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero.  The range check covers the per-lane (vector) offset, so every
// row offset goes there; the scalar offset argument of dma16 stays 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS at lds + 16 * lane
// (buffer_load_dwordx4 ... lds).  The builtin only exists for the device
// target, so the host pass of the single-source compile sees an empty body.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
#else
  (void)r, (void)lds, (void)voff;
#endif
}

// The same load issued from inline assembly, for pipelines that keep several
// loads in flight while they read other LDS buffers.  The LDS address and the
// resource must be wave-uniform (they are taken from the first active lane).  The compiler does not see
// this as an LDS write (so it inserts no wait before unrelated LDS reads); the
// caller waits with wait_vmcnt before it reads the bytes.  The resource is
// passed as four dwords: base (48 bits), stride 0, num_records, flags.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc_words(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane(int(uint32_t(a))),
               __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}
__device__ __forceinline__ void dma16_async(i32x4 r, char* lds, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m), "v"(voff), "s"(r) : "memory");
#else
  (void)r, (void)lds, (void)voff;
#endif
}

// dma16_async with the LDS address given as a wave-uniform 32-bit LDS byte
// address plus a compile-time offset, added into m0 by the same instruction
// sequence (one scalar add per load; no generic-to-LDS pointer conversion).
template <int kOff>
__device__ __forceinline__ void dma16_async_at(i32x4 r, uint32_t lds_addr, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_add_u32 m0, %0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds" ::"s"(lds_addr), "i"(kOff), "v"(voff),
               "s"(r)
               : "memory");
#else
  (void)r, (void)lds_addr, (void)voff;
#endif
}
// kN consecutive 1 KB wave loads: load u fills LDS [lds_addr + kOff + 1024 u,
// + 1024) from per-lane offset voff[u]
template <int kOff, int kN, int kU = 0>
__device__ __forceinline__ void dma16_async_run(i32x4 r, uint32_t lds_addr, const int* voff) {
  if constexpr (kU < kN) {
    dma16_async_at<kOff + kU * 1024>(r, lds_addr, voff[kU]);
    dma16_async_run<kOff, kN, kU + 1>(r, lds_addr, voff);
  }
}

// dma16_async with the non-temporal cache policy (nt), for data read exactly
// once: the lines are not kept for reuse.  A streaming read of HBM runs about
// 13% faster this way on gfx950 (7.0 against 6.2 TB/s for a plain grid-stride
// read of 2 GiB), so the decode kernels, which touch every byte once, use it.
__device__ __forceinline__ void dma16_stream(i32x4 r, char* lds, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds)));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(m), "v"(voff), "s"(r) : "memory");
#else
  (void)r, (void)lds, (void)voff;
#endif
}

// s_waitcnt vmcnt(n) with lgkmcnt and expcnt left free (gfx9 encoding: vmcnt
// bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Exact integer budget rule: k = min(n, max(min_blocks, ceil(ratio_q16 * n / 2^16))).
__host__ __device__ __forceinline__ int budget_blocks(int n, int min_blocks, uint32_t ratio_q16) {
  long long want = ((long long)ratio_q16 * (long long)n + 65535ll) >> 16;
  if (want < min_blocks) want = min_blocks;
  return want < n ? int(want) : n;
}

}  // namespace sa
