// Block attention mass for offline budget calibration (gfx950, bf16).
//
// W[b][h][m][n] = sum over the query rows t of block m of head h of their exact
// causal softmax probabilities on the keys of block n (n <= m; zero above).
// This is the attention weight the per-head budgets are calibrated on: a head's
// budget is the one whose best block selection keeps a target share of it, and
// the max-min shifting moves budget between heads by it ("S-HPLB: Efficient LLM
// Attention Serving via Sparsity-Aware Head Parallelism Load Balance", Italian
// summary §2.A, Chinese summary §2.1).
//
// One workgroup per (b, h, m), four waves, wave w owns query rows 32w..32w+31.
// Two passes over the key blocks 0..m, each staged through LDS:
//   pass 1  S^T = K Q^T on the MFMA pipe; running row max and sum -> the row's
//           log2-sum-exp L (the two half-waves' partial states merged at the end);
//   pass 2  S^T again; sum of exp2(S * scale * log2(e) - L) over the block's
//           visible (query, key) pairs, reduced over the workgroup in a fixed
//           order (no atomics, bitwise reproducible).
// Calibration is offline, so the kernel favours plainness over speed: no
// pipelining, plain global loads into LDS.

#include "sa_device.hpp"
#include "sa_kernels.hpp"

namespace sa {

namespace {

constexpr int kMB = 128;  // block size

template <int D>
__global__ __launch_bounds__(256) void block_mass_kernel(MassParams p) {
  constexpr int kRow = D * 2;        // bytes per K row
  constexpr int kCpr = kRow / 16;    // 16-byte chunks per row
  constexpr int kDG = D / 16;        // k-groups of the 32x32x16 MFMA
  constexpr int kKMask = (kCpr < 16 ? kCpr : 16) - 1;
  __shared__ __attribute__((aligned(16))) char ks[kMB * kRow];
  __shared__ float red[4];

  const int m = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;
  const int qrow = m * kMB + wave * 32 + col;
  const bool row_ok = qrow < S;
  const float c2 = p.scale_log2;
  auto swz = [](int r) { return (r / (kRow >= 256 ? 1 : 256 / kRow)) & kKMask; };

  // Q^T fragments: lane half g holds d = 16 dg + 8 g .. +7 of query qrow
  u32x4 qf[kDG];
  {
    const char* rp = reinterpret_cast<const char*>(p.q) +
                     (bi * p.qs0 + h * p.qs1 + (int64_t)(row_ok ? qrow : 0) * p.qs2) * 2;
#pragma unroll
    for (int dg = 0; dg < kDG; ++dg)
      qf[dg] = row_ok ? *reinterpret_cast<const u32x4*>(rp + (dg * 16 + half * 8) * 2) : u32x4{0u, 0u, 0u, 0u};
  }
  const char* kbase = reinterpret_cast<const char*>(p.k) + (bi * p.ks0 + (h / p.G) * p.ks1) * 2;

  // K rows of block n into LDS (rows past the sequence end as zero)
  auto load_k = [&](int n) {
    __syncthreads();  // the previous block's reads are done
    for (int c = tid; c < kMB * kCpr; c += 256) {
      const int r = c / kCpr, cc = c % kCpr;
      const int row = n * kMB + r;
      const u32x4 v = row < S ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)row * p.ks2 * 2 + cc * 16)
                              : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(ks + r * kRow + ((cc ^ swz(r)) * 16)) = v;
    }
    __syncthreads();
  };
  // S^T of one 32-key tile kt: element i of this lane is key 32 kt + 8 (i / 4)
  // + 4 half + i % 4 of the block against query qrow
  auto tile = [&](int kt) {
    f32x16 s = f32x16{};
    const int r = kt * 32 + col;
#pragma unroll
    for (int dg = 0; dg < kDG; ++dg) {
      const u32x4 a = lds16(ks, r * kRow + ((dg * 2 + half) ^ swz(r)) * 16);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[dg]),
                                                  s, 0, 0, 0);
    }
    return s;
  };
  auto visible = [&](int n, int kt, int i) {
    const int key = n * kMB + kt * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
    return row_ok && key <= qrow;
  };

  // pass 1: log2-sum-exp of every query row over keys 0..qrow
  float mx = kNegInf, l = 0.f;
  for (int n = 0; n <= m; ++n) {
    load_k(n);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x16 s = tile(kt);
      float tm = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = visible(n, kt, i) ? s[i] * c2 : kNegInf;
        tm = fmaxf(tm, s[i]);
      }
      const float mn = fmaxf(mx, tm);
      if (mn != kNegInf) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += __builtin_amdgcn_exp2f(s[i] - mn);
        l = l * __builtin_amdgcn_exp2f(mx - mn) + acc;
        mx = mn;
      }
    }
  }
  // merge the two half-waves' states of the same query
  {
    const float mo = __shfl_xor(mx, 32, 64), lo = __shfl_xor(l, 32, 64);
    const float mm = fmaxf(mx, mo);
    l = (mx == kNegInf ? 0.f : l * __builtin_amdgcn_exp2f(mx - mm)) +
        (mo == kNegInf ? 0.f : lo * __builtin_amdgcn_exp2f(mo - mm));
    mx = mm;
  }
  const float L = mx + __log2f(l);  // -inf for rows past the end

  // pass 2: probability mass on each key block
  float* const out = p.mass + (((int64_t)bi * p.Hq + h) * p.NB + m) * p.NB;
  for (int n = 0; n <= m; ++n) {
    load_k(n);
    float acc = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const f32x16 s = tile(kt);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc += visible(n, kt, i) ? __builtin_amdgcn_exp2f(s[i] * c2 - L) : 0.f;
    }
    acc = wave_sum(acc);
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (tid == 0) out[n] = (red[0] + red[1]) + (red[2] + red[3]);
  }
  for (int n = m + 1 + tid; n < p.NB; n += 256) out[n] = 0.f;
}

// Output deviation of query head h = blockIdx.x: sqrt(sum (a - r)^2) /
// sqrt(sum r^2) over every sequence, row and channel of the head, the output
// moved by a budget against dense attention ("Fluxion", Italian summary,
// Intuizioni Chiave 1).  Each thread sums a fixed share of the 16-byte chunks
// in double; the workgroup reduces in a fixed tree order (bitwise reproducible).
__global__ __launch_bounds__(256) void output_deviation_kernel(DeviationParams p) {
  __shared__ double red[2][256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int cpr = p.D / 4;  // 16-byte chunks per row
  const int64_t per_seq = (int64_t)p.S * cpr;
  double num = 0.0, den = 0.0;
  for (int bi = 0; bi < p.batch; ++bi) {
    const float* ab = p.a + bi * p.s0 + h * p.s1;
    const float* rb = p.r + bi * p.s0 + h * p.s1;
    for (int64_t c = tid; c < per_seq; c += 256) {
      const int64_t row = c / cpr;
      const int col = int(c % cpr) * 4;
      const f32x4 av = *reinterpret_cast<const f32x4*>(ab + row * p.s2 + col);
      const f32x4 rv = *reinterpret_cast<const f32x4*>(rb + row * p.s2 + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d = (double)av[e] - (double)rv[e];
        num += d * d;
        den += (double)rv[e] * (double)rv[e];
      }
    }
  }
  red[0][tid] = num;
  red[1][tid] = den;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      red[0][tid] += red[0][tid + w];
      red[1][tid] += red[1][tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) p.dev[h] = red[1][0] > 0.0 ? sqrt(red[0][0]) / sqrt(red[1][0]) : 0.0;
}

}  // namespace

hipError_t launch_output_deviation(const DeviationParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(output_deviation_kernel, dim3(p.Hq), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_block_mass(const MassParams& p, int D, int batch, hipStream_t stream) {
  dim3 grid(p.NB, p.Hq, batch);
  if (D == 128) hipLaunchKernelGGL(block_mass_kernel<128>, grid, dim3(256), 0, stream, p);
  else if (D == 64) hipLaunchKernelGGL(block_mass_kernel<64>, grid, dim3(256), 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
