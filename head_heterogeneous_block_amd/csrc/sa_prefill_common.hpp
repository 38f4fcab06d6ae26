// Definitions of the block-sparse prefill attention kernel (sa_prefill.hip):
// its tile and step geometry, LDS swizzles, the step record of its cursor and
// the reader of rarely used kernel arguments.
#pragma once

#include <cstddef>

#include "sa_device.hpp"
#include "sa_kernels.hpp"

namespace sa {
namespace prefill {

constexpr int kKS = 64;       // keys per step
// log2 headroom before the running max is raised (P <= 2^kLazy).  P is
// rounded to bf16 for the P V MFMAs (relative error up to 2^-8), and the
// normaliser sums those same rounded values, so the output is an exact convex
// combination of the V rows under slightly perturbed weights whatever the
// headroom: the largest P of a row being rounded too no longer biases it.  (A
// normaliser over the unrounded P left an error of up to 2^-8 of the dominant
// key's V row when one key held most of a row's weight.)  A large headroom
// keeps the rescaling of O rare.
constexpr float kLazy = 8.f;

// swap bits 2 and 3 of a key index (an involution)
__device__ __forceinline__ int perm_key(int k) { return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <typename T, int D, int B>
struct Cfg {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kW = B / 32;  // waves, 32 queries each
  static constexpr int kThreads = 64 * kW;
  static constexpr int kE16 = 16 / int(sizeof(T));  // elements per 16 bytes
  static constexpr int kNSub = B / kKS;
  static constexpr int kDT = D / 32;  // 32-row d tiles of O^T
  static constexpr int kRow = D * int(sizeof(T));  // bytes per K or V row
  static constexpr int kCpr = kRow / 16;           // 16-byte chunks per row
  static constexpr int kTile = kKS * kRow;         // bytes of one K (or V) step
  static constexpr int kInsts = kTile / 1024;      // 1 KB direct-to-LDS wave instructions per tile
  static constexpr int kInstsPerWave = kInsts / kW;
  static constexpr int kDG = D / (2 * kE16);  // Q K^T k-groups of 16 bytes per lane
  static constexpr int kLds = 4 * kTile;      // K ring (2) + V ring (2)
  static_assert(kInsts % kW == 0, "direct loads must split evenly over the waves");

  // 16-byte chunk swizzles, free of bank conflicts whether the LDS serves 128
  // or 256 bytes per clock.  K rows (read 16 B per lane, one row per lane):
  // the 16 rows a 256-byte cycle touches land on 16 distinct slots.  V rows
  // (transposed 8-byte reads, 4 rows x 2 or 4 chunks per cycle): the XOR
  // patterns {0, 6, 10, 12} differ both in chunk bits 1-2 and in bits 2-3.
  static constexpr int kRowsPer256 = kRow >= 256 ? 1 : 256 / kRow;
  static constexpr int kKMask = (kCpr < 16 ? kCpr : 16) - 1;
  __device__ static int swz_k(int row) { return (row / kRowsPer256) & kKMask; }
  __device__ static int swz_v(int row) {
    const int x = (0xCA60 >> ((row & 3) * 4)) & 15;  // 0, 6, 10, 12
    return x & (kCpr - 1);
  }
};

// One 64-key step, wave-uniform (scalar registers).
struct Step {
  int valid;
  int item;  // position in the bin's item list
  int j;     // position in the tile's block list
  int hs;    // 64-key step within the key block
  int n;     // key block index
  int tile;  // (b * Hq + h) * NB + m
  int m;     // query block of the tile
  int bh;    // b * Hq + h
  int kvs;   // (batch << 16) | KV head of the tile
};

// A field of the kernel's only argument, read from the kernel-argument
// segment (scalar cache) where it is used.  Fields needed only when a tile
// starts or ends, or when a schedule window is refilled, are read this way so
// that they do not hold scalar registers through the persistent loop; the
// empty asm makes the pointer opaque, so the load is not hoisted out of it.
template <typename F>
__device__ __forceinline__ F kernel_arg(int offset) {
  auto kp = (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return *(const __attribute__((address_space(4))) F*)(kp + offset);
}
#define COLD(field) kernel_arg<decltype(PrefillParams::field)>(offsetof(PrefillParams, field))

// Start (which = 0) or end (1) stamp of this workgroup on the constant clock,
// when the launch records them: one lane writes it with a vector store.
__device__ __forceinline__ void wg_stamp(int which) {
  uint64_t* const t = COLD(wg_times);
  if (t == nullptr) return;
  const uint64_t now = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    __builtin_nontemporal_store(now, t + 2 * blockIdx.x + which);
  }
}


}  // namespace prefill
}  // namespace sa
