// Measurement kernels for the roofline denominators on the GPU at hand: the
// bf16 MFMA rate and the HBM streaming-read rate the chip actually sustains,
// reported beside the published peaks (2.5 PFLOP/s dense bf16, 8 TB/s).
//
//   mfma_peak_kernel : every wave runs kChains independent accumulation chains
//                      of v_mfma_f32_32x32x16_bf16, so the pipe never waits on
//                      a result.  Operands of ones (each accumulator element
//                      ends at exactly 16 * iters), or pseudo-random bf16
//                      values in [-1, 1): four A and four B fragments per lane,
//                      chain c multiplying A[c % 4] by B[c % 4].  The chip
//                      draws more power multiplying random mantissas, and its
//                      power limit then lowers the clock, so the random
//                      operands give the rate matrix work on real data can
//                      reach.
//   hbm_read_kernel  : grid-stride 16-byte non-temporal loads over a buffer,
//                      eight in flight per thread, XOR-reduced into one word
//                      per thread so no load is dead.
// Neither kernel reads or writes outside the buffers it is given.

#include "sa_device.hpp"
#include "sa_kernels.hpp"

namespace sa {

namespace {

constexpr int kChains = 8;
constexpr int kInFlight = 8;  // 16-byte loads per thread in flight

// The "lowbias32" 32-bit integer hash (C. Wellons, "Prospecting for Hash
// Functions"): element e of operand fragment f of global thread t is
// bf16(((h & 0xffff) - 32768) / 32768) with h = hash(64 t + 8 f + e); the
// quotient is exact in fp32 and rounds to nearest-even into bf16.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__device__ __forceinline__ bf16x8 probe_frag(uint32_t t, int f) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    r[e] = (__bf16)((float)((int)(probe_hash(64u * t + 8u * f + e) & 0xffffu) - 32768) * (1.f / 32768.f));
  return r;
}

template <bool kRandom>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if constexpr (kRandom) {
      a[f] = probe_frag(t, f);
      b[f] = probe_frag(t, 4 + f);
    } else {
      a[f] = bf16x8{(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                    (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
      b[f] = a[f];
    }
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c % 4], b[c % 4], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][c];
  sink[t] = s;
}

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* src, int64_t n16, uint32_t* sink) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t x = 0u;
  int64_t i = tid;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 a[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) a[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) x ^= a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  sink[tid] = x;
}

}  // namespace

hipError_t launch_mfma_peak(int n_workgroups, int iters, bool random_operands, float* sink, hipStream_t stream) {
  if (random_operands) hipLaunchKernelGGL(mfma_peak_kernel<true>, dim3(n_workgroups), dim3(256), 0, stream, iters, sink);
  else hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3(n_workgroups), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

hipError_t launch_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int n_workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(n_workgroups), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace sa
