// Block-sparse decode attention for gfx950.
//
// One query token per (sequence, query head) attends to the tokens of its own
// selected blocks, each head at its own block granularity (streaming heads keep
// sink + recent blocks, retrieval heads a scored top-k: "Fluxion", Italian
// summary, Intuizioni Chiave 2).  GQA is handled at KV-group level (same page,
// Componenti di Sistema): the selections of the query heads that share a KV
// head are merged into one sorted list of 16-token atoms, each tagged with the
// mask of heads that want it, so every K/V byte of the group is read from HBM
// once per step.  Decode is bound by data movement, so the kernels are built
// for streaming HBM bandwidth:
//
//   plan    : per (sequence, KV head) the union atom list (LDS bitmaps, ordered
//             compaction).
//   attend  : split-KV over chunks of the atom list; lanes own (token, d-slice)
//             pairs, keep an online-softmax state per head, and the states are
//             merged inside the wave, then across waves; one partial
//             (max, sum, o) per (chunk, head).
//   combine : fixed-order merge of the chunk partials per (sequence, head).
// No floating-point atomics: results are bitwise reproducible.

#include "sa_device.hpp"
#include "sa_kernels.hpp"

namespace sa {

namespace {

// ---------------------------------------------------------------- plan
constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodePlanParams p) {
  extern __shared__ uint32_t bits[];  // [G][n_words]
  const int j = blockIdx.x, bi = blockIdx.y;
  const int tid = threadIdx.x;
  const int n_words = (p.n_atoms + 31) / 32;
  for (int i = tid; i < p.G * n_words; i += kPlanThreads) bits[i] = 0u;
  __syncthreads();
  for (int gi = 0; gi < p.G; ++gi) {
    const int h = j * p.G + gi;
    const int g = p.heads.gran[h];
    const int apb = g / kAtom;  // atoms per block
    const int cnt = p.block_cnt[(int64_t)bi * p.Hq + h];
    const int32_t* idx = p.block_idx + ((int64_t)bi * p.Hq + h) * p.kmax;
    uint32_t* w = bits + gi * n_words;
    for (int t = tid; t < cnt * apb; t += kPlanThreads) {
      const int n = idx[t / apb];
      const int a = n * apb + t % apb;
      if (n >= 0 && a < p.n_atoms) atomicOr(&w[a >> 5], 1u << (a & 31));
    }
  }
  __syncthreads();
  // ordered compaction of the union, 32 atoms (one word) per thread per pass
  __shared__ uint32_t wave_tot[kPlanThreads / 64];
  __shared__ uint32_t base_s;
  if (tid == 0) base_s = 0;
  __syncthreads();
  uint32_t* out = p.atoms + ((int64_t)bi * p.Hkv + j) * p.max_union;
  for (int w0 = 0; w0 < n_words; w0 += kPlanThreads) {
    const int wi = w0 + tid;
    uint32_t u = 0;
    if (wi < n_words)
      for (int gi = 0; gi < p.G; ++gi) u |= bits[gi * n_words + wi];
    const uint32_t c = __popc(u);
    // exclusive scan of c across the block
    uint32_t x = c;
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[wv] = x;
    __syncthreads();
    uint32_t off = base_s;
    for (int i = 0; i < wv; ++i) off += wave_tot[i];
    off += x - c;
    uint32_t rem = u;
    while (rem) {
      const int b = __ffs(rem) - 1;
      rem &= rem - 1;
      const int a = wi * 32 + b;
      uint32_t mask = 0;
      for (int gi = 0; gi < p.G; ++gi) mask |= ((bits[gi * n_words + wi] >> b) & 1u) << gi;
      if (off < (uint32_t)p.max_union) out[off] = uint32_t(a) | (mask << 24);
      ++off;
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) {
      uint32_t tot = 0;
      for (int i = 0; i < kPlanThreads / 64; ++i) tot += wave_tot[i];
      base_s += tot;
    }
    __syncthreads();
  }
  if (tid == 0) p.n_union[(int64_t)bi * p.Hkv + j] = min<int>(base_s, p.max_union);
}

// ---------------------------------------------------------------- attend
// LPT lanes per token, DS = D / LPT d-values per lane, GM = max heads per group.
template <typename T, int D, int LPT, int GM>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeAttnParams p) {
  constexpr int DS = D / LPT;
  constexpr int TPP = 64 / LPT;           // tokens per wave pass
  constexpr int PPA = kAtom / TPP;        // passes per atom
  constexpr int kE16 = 16 / int(sizeof(T));
  constexpr int NLD = DS / kE16;          // 16-byte loads per lane per tensor
  const int c = blockIdx.x, j = blockIdx.y, bi = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nu = p.n_union[(int64_t)bi * p.Hkv + j];
  const int a_beg = c * p.chunk_atoms;
  if (a_beg >= nu) return;
  const int a_end = min(nu, a_beg + p.chunk_atoms);
  const uint32_t* atoms = p.atoms + ((int64_t)bi * p.Hkv + j) * p.max_union;
  const int tl = lane / LPT, sl = lane % LPT;
  const int d0 = sl * DS;

  float qv[GM][DS];
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    if (gi < p.G) {
      const char* qrow = reinterpret_cast<const char*>(p.q) + (bi * p.qs0 + (j * p.G + gi) * p.qs1) * (int64_t)sizeof(T);
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        float x;
        if constexpr (sizeof(T) == 2) x = bf16_to_f32(reinterpret_cast<const bf16_t*>(qrow)[d0 + e]);
        else x = reinterpret_cast<const float*>(qrow)[d0 + e];
        qv[gi][e] = x * p.scale_log2;
      }
    }
  }
  float m_[GM], l_[GM], o_[GM][DS];
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    m_[gi] = kNegInf;
    l_[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < DS; ++e) o_[gi][e] = 0.f;
  }

  const char* kbase = reinterpret_cast<const char*>(p.k) + (bi * p.ks0 + j * p.ks1) * (int64_t)sizeof(T);
  const char* vbase = reinterpret_cast<const char*>(p.v) + (bi * p.vs0 + j * p.vs1) * (int64_t)sizeof(T);
  const int64_t krs = p.ks2 * (int64_t)sizeof(T), vrs = p.vs2 * (int64_t)sizeof(T);

  // passes of this wave: pass index u over the chunk's (atom, sub-pass) pairs
  const int n_pass = (a_end - a_beg) * PPA;
  u32x4 kr[2][NLD], vr[2][NLD];
  uint32_t meta[2];
  int tok[2];
  auto issue = [&](int u, int slot) {
    const int ai = a_beg + u / PPA;
    const uint32_t at = atoms[ai];
    const int t = int(at & 0xffffffu) * kAtom + (u % PPA) * TPP + tl;
    meta[slot] = at >> 24;
    tok[slot] = t;
    const bool ok = t < p.kv_len;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kr[slot][i] = ok ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)t * krs + (d0 + i * kE16) * (int)sizeof(T))
                       : u32x4{0u, 0u, 0u, 0u};
      vr[slot][i] = ok ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)t * vrs + (d0 + i * kE16) * (int)sizeof(T))
                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  int u = wave;
  if (u < n_pass) issue(u, 0);
  int slot = 0;
  for (; u < n_pass; u += 4) {
    if (u + 4 < n_pass) issue(u + 4, slot ^ 1);
    float kf[DS], vf[DS];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (sizeof(T) == 2) {
          kf[i * 8 + 2 * w] = bf16_lo(kr[slot][i][w]);
          kf[i * 8 + 2 * w + 1] = bf16_hi(kr[slot][i][w]);
          vf[i * 8 + 2 * w] = bf16_lo(vr[slot][i][w]);
          vf[i * 8 + 2 * w + 1] = bf16_hi(vr[slot][i][w]);
        } else {
          kf[i * 4 + w] = __uint_as_float(kr[slot][i][w]);
          vf[i * 4 + w] = __uint_as_float(vr[slot][i][w]);
        }
      }
    }
    const uint32_t mask = meta[slot];
    const bool in_range = tok[slot] < p.kv_len;
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      if (!((mask >> gi) & 1u)) continue;  // uniform across the wave (one atom per pass)
      float z = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) z = fmaf(qv[gi][e], kf[e], z);
#pragma unroll
      for (int o = 1; o < LPT; o <<= 1) z += __shfl_xor(z, o, 64);
      if (!in_range) z = kNegInf;
      const float m_new = fmaxf(m_[gi], z);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_[gi] - m_use);
      const float pz = __builtin_amdgcn_exp2f(z - m_use);
      m_[gi] = m_new;
      l_[gi] = l_[gi] * alpha + pz;
#pragma unroll
      for (int e = 0; e < DS; ++e) o_[gi][e] = fmaf(o_[gi][e], alpha, pz * vf[e]);
    }
    slot ^= 1;
  }

  // merge the per-lane states over the token lanes of the wave (lane bits
  // above the d-slice bits)
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    if (gi >= p.G) break;
#pragma unroll
    for (int o = LPT; o < 64; o <<= 1) {
      const float mo = __shfl_xor(m_[gi], o, 64);
      const float lo = __shfl_xor(l_[gi], o, 64);
      const float mn = fmaxf(m_[gi], mo);
      const float mu = mn == kNegInf ? 0.f : mn;
      const float a = __builtin_amdgcn_exp2f(m_[gi] - mu), b = __builtin_amdgcn_exp2f(mo - mu);
      l_[gi] = l_[gi] * a + lo * b;
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        const float oo = __shfl_xor(o_[gi][e], o, 64);
        o_[gi][e] = o_[gi][e] * a + oo * b;
      }
      m_[gi] = mn;
    }
  }
  // merge the 4 waves through LDS: lanes 0..LPT-1 of each wave hold the wave's state
  __shared__ float so[4][GM][D];
  __shared__ float sm[4][GM][2];
  if (tl == 0) {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      if (gi >= p.G) break;
#pragma unroll
      for (int e = 0; e < DS; ++e) so[wave][gi][d0 + e] = o_[gi][e];
      if (sl == 0) {
        sm[wave][gi][0] = m_[gi];
        sm[wave][gi][1] = l_[gi];
      }
    }
  }
  __syncthreads();
  const int64_t pbase = (((int64_t)bi * p.Hkv + j) * p.n_chunks + c) * p.G;
  for (int i = tid; i < p.G * D; i += 256) {
    const int gi = i / D, d = i % D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, sm[w][gi][0]);
    const float mu = mx == kNegInf ? 0.f : mx;
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm[w][gi][0] - mu);
      acc += so[w][gi][d] * f;
      l += sm[w][gi][1] * f;
    }
    p.part_o[(pbase + gi) * D + d] = acc;
    if (d == 0) {
      p.part_ml[(pbase + gi) * 2 + 0] = mx;
      p.part_ml[(pbase + gi) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------- combine
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeCombineParams p, int dtype) {
  const int h = blockIdx.x, bi = blockIdx.y;
  const int j = h / p.G, gi = h % p.G;
  const int d = threadIdx.x;
  const int nu = p.n_union[(int64_t)bi * p.Hkv + j];
  const int nch = (nu + p.chunk_atoms - 1) / p.chunk_atoms;
  const int64_t base = ((int64_t)bi * p.Hkv + j) * p.n_chunks;
  float mx = kNegInf;
  for (int c = 0; c < nch; ++c) mx = fmaxf(mx, p.part_ml[((base + c) * p.G + gi) * 2]);
  const float mu = mx == kNegInf ? 0.f : mx;
  float acc = 0.f, l = 0.f;
  for (int c = 0; c < nch; ++c) {
    const int64_t r = (base + c) * p.G + gi;
    const float f = __builtin_amdgcn_exp2f(p.part_ml[r * 2] - mu);
    acc += p.part_o[r * D + d] * f;
    l += p.part_ml[r * 2 + 1] * f;
  }
  const float o = l > 0.f ? acc / l : 0.f;
  const int64_t oi = bi * p.os0 + h * p.os1 + d;
  if (p.out_f32 || dtype == 1) reinterpret_cast<float*>(p.o)[oi] = o;
  else reinterpret_cast<bf16_t*>(p.o)[oi] = bf16_t(pack_bf16x2(o, 0.f) & 0xffffu);
  if (p.lse && d == 0) p.lse[(int64_t)bi * p.Hq + h] = l > 0.f ? (mx + __log2f(l)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_decode_plan(const DecodePlanParams& p, int batch, hipStream_t stream) {
  const size_t lds = size_t(p.G) * ((p.n_atoms + 31) / 32) * 4;
  hipLaunchKernelGGL(decode_plan_kernel, dim3(p.Hkv, batch), dim3(kPlanThreads), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const DecodeAttnParams& p, int dtype, int D, int batch, hipStream_t stream) {
  dim3 grid(p.n_chunks, p.Hkv, batch);
  if (dtype == 0) {
    if (D == 128 && p.G <= 4) hipLaunchKernelGGL((decode_attn_kernel<bf16_t, 128, 4, 4>), grid, dim3(256), 0, stream, p);
    else if (D == 128 && p.G <= 8) hipLaunchKernelGGL((decode_attn_kernel<bf16_t, 128, 8, 8>), grid, dim3(256), 0, stream, p);
    else if (D == 64 && p.G <= 8) hipLaunchKernelGGL((decode_attn_kernel<bf16_t, 64, 4, 8>), grid, dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
  } else {
    if (D == 128 && p.G <= 4) hipLaunchKernelGGL((decode_attn_kernel<float, 128, 4, 4>), grid, dim3(256), 0, stream, p);
    else if (D == 128 && p.G <= 8) hipLaunchKernelGGL((decode_attn_kernel<float, 128, 8, 8>), grid, dim3(256), 0, stream, p);
    else if (D == 64 && p.G <= 8) hipLaunchKernelGGL((decode_attn_kernel<float, 64, 4, 8>), grid, dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeCombineParams& p, int dtype, int D, int batch, hipStream_t stream) {
  dim3 grid(p.Hq, batch);
  if (D == 128) hipLaunchKernelGGL((decode_combine_kernel<128>), grid, dim3(128), 0, stream, p, dtype);
  else if (D == 64) hipLaunchKernelGGL((decode_combine_kernel<64>), grid, dim3(64), 0, stream, p, dtype);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
