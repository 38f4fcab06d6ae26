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

#include <type_traits>

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
  // Every selected block sets its atoms' bits: a block of g = 16 * apb tokens
  // covers apb consecutive atoms, all in one 32-bit word (apb divides 32 and
  // the block starts at a multiple of apb).  The block counts and the block
  // indices of all heads of a round are loaded together (the indices do not
  // wait for the counts), and the bitmaps are cleared while they are in flight.
  constexpr int kGM = 8;  // heads per group, at most
  constexpr int kR = 2;   // rounds of kPlanThreads blocks per head in one batch of loads
  int cnt[kGM], apb[kGM];
#pragma unroll
  for (int gi = 0; gi < kGM; ++gi) {
    const int h = j * p.G + (gi < p.G ? gi : 0);
    cnt[gi] = gi < p.G ? p.block_cnt[(int64_t)bi * p.Hq + h] : 0;
    apb[gi] = p.heads.gran[h] / kAtom;
  }
  int nv[kR][kGM];
  auto load = [&](int b0) {
#pragma unroll
    for (int r = 0; r < kR; ++r)
#pragma unroll
      for (int gi = 0; gi < kGM; ++gi) {
        const int b = b0 + r * kPlanThreads + tid;
        nv[r][gi] = gi < p.G && b < p.kmax ? p.block_idx[((int64_t)bi * p.Hq + j * p.G + gi) * p.kmax + b] : -1;
      }
  };
  load(0);
  for (int i = tid; i < p.G * n_words; i += kPlanThreads) bits[i] = 0u;
  __syncthreads();
  for (int b0 = 0; b0 < p.kmax; b0 += kR * kPlanThreads) {
    if (b0 > 0) load(b0);
#pragma unroll
    for (int r = 0; r < kR; ++r)
#pragma unroll
      for (int gi = 0; gi < kGM; ++gi) {
        const int b = b0 + r * kPlanThreads + tid;
        // out-of-range indices (n >= n_atoms can never be a block of the cache)
        // are skipped before n * apb could overflow
        if (b >= cnt[gi] || nv[r][gi] < 0 || nv[r][gi] >= p.n_atoms) continue;
        const int a = nv[r][gi] * apb[gi];
        const int na = min(apb[gi], p.n_atoms - a);
        if (na > 0) atomicOr(&bits[gi * n_words + (a >> 5)], ((na >= 32 ? 0u : (1u << na)) - 1u) << (a & 31));
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
    uint32_t hw[kGM], u = 0;  // this word of every head's bitmap, and their union
#pragma unroll
    for (int gi = 0; gi < kGM; ++gi) {
      hw[gi] = wi < n_words && gi < p.G ? bits[gi * n_words + wi] : 0u;
      u |= hw[gi];
    }
    const uint32_t c = __popc(u);
    // exclusive scan of c across the block
    const uint32_t x = wave_scan_incl(c);
    const int lane = tid & 63, wv = tid >> 6;
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
#pragma unroll
      for (int gi = 0; gi < kGM; ++gi) mask |= ((hw[gi] >> b) & 1u) << gi;
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
    if (d == 0) {  // fp32 probabilities: nothing is rounded
      p.part_ml[(pbase + gi) * kPartMl + 0] = mx;
      p.part_ml[(pbase + gi) * kPartMl + 1] = l;
      p.part_ml[(pbase + gi) * kPartMl + 2] = l;
    }
  }
}

// ---------------------------------------------------------------- attend, bf16 on MFMA
// One wave per workgroup and per chunk of the union atom list.  The wave
// streams its atoms through a ring of kDStages LDS stages (one stage = K and V
// rows of one 16-token atom, gathered with direct-to-LDS buffer loads, so
// three atoms are in flight while one is computed) and keeps no barrier.
// Per atom, with the group's query heads as the MFMA columns (zero beyond G):
//   S^T[key][head] = K Q^T   v_mfma_f32_16x16x32_bf16: A = K rows (LDS,
//                            16 bytes per lane), B = Q^T (registers);
//                            lane element i <-> key 4*(lane/16) + i.
//   O^T[d][head] += V^T P^T  v_mfma_f32_16x16x16_bf16: A = V^T read with
//                            ds_read_b64_tr_b16, B = P^T straight from the
//                            S^T accumulators (same key <-> lane layout).
// Keys whose atom a head did not select, and tokens past the cache end, get
// probability 0.  Softmax in the log2 domain with a lazily raised running max
// (raised only when a score beats it by more than 2^kLazy), as in prefill.
constexpr int kDStages = 4;
constexpr float kDLazy = 8.f;

template <int D>
struct DCfg {
  static constexpr int kRow = D * 2;                 // bytes per K or V row
  static constexpr int kCpr = kRow / 16;             // 16-byte chunks per row
  static constexpr int kAtomBytes = kAtom * kRow;    // one tensor's rows of an atom
  static constexpr int kInsts = kAtomBytes / 1024;   // 1 KB direct loads per tensor and atom
  static constexpr int kDK = D / 32;                 // k-steps of Q K^T
  static constexpr int kDT = D / 16;                 // d-tiles of O^T
  static constexpr int kRowsPer256 = kRow >= 256 ? 1 : 256 / kRow;
  static constexpr int kKMask = (kCpr < 16 ? kCpr : 16) - 1;
  // K (16-byte reads, 16 rows per group of lanes) and V (transposed 8-byte
  // reads of 32-byte row pieces, 4 rows per group): the swizzles spread the
  // rows read together over distinct LDS banks; V's is even, so the two
  // 16-byte halves of a 32-byte piece stay adjacent.
  __device__ static int swz_k(int row) { return (row / kRowsPer256) & kKMask; }
  __device__ static int swz_v(int row) { return (2 * (row / kRowsPer256)) & (kCpr - 1); }
  static_assert(kInsts * 1024 == kAtomBytes, "atom rows must fill whole 1 KB loads");
};

template <int D>
__global__ __launch_bounds__(64) void decode_attn_mfma_kernel(DecodeAttnParams p) {
  using C = DCfg<D>;
  // LDS ring: one variable per stage (K and V rows of one atom each)
  __shared__ __attribute__((aligned(1024))) char k0[C::kAtomBytes], k1[C::kAtomBytes], k2[C::kAtomBytes],
      k3[C::kAtomBytes];
  __shared__ __attribute__((aligned(1024))) char v0[C::kAtomBytes], v1[C::kAtomBytes], v2[C::kAtomBytes],
      v3[C::kAtomBytes];
  static_assert(kDStages == 4, "stage variables");

  const int c = blockIdx.x, j = blockIdx.y, bi = blockIdx.z;
  const int lane = threadIdx.x;
  const int col = lane & 15;  // MFMA column (query head of the group) / A row
  const int qg = lane >> 4;   // 16-lane group: k-group of A/B, row group of the output
  const int nu = p.n_union[(int64_t)bi * p.Hkv + j];
  const int a_beg = c * p.chunk_atoms;
  if (a_beg >= nu) return;
  const int na = min(nu - a_beg, p.chunk_atoms);  // <= 64
  const uint32_t aw = lane < na ? p.atoms[((int64_t)bi * p.Hkv + j) * p.max_union + a_beg + lane] : 0u;

  // Q^T fragments: lane holds head `col`, d = 32 s + 8 qg .. +7
  u32x4 qf[C::kDK];
  {
    const bool ok = col < p.G;
    const bf16_t* qrow = reinterpret_cast<const bf16_t*>(p.q) + bi * p.qs0 + (j * p.G + (ok ? col : 0)) * p.qs1;
#pragma unroll
    for (int s = 0; s < C::kDK; ++s)
      qf[s] = ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * qg) : u32x4{0u, 0u, 0u, 0u};
  }

  const int krs = int(p.ks2 * 2), vrs = int(p.vs2 * 2);
  // The buffer is the (sequence, KV head) slice of the cache, or with pages the
  // KV head's page pool; arow (lane l: atom a_beg + l) is the row of the atom's
  // first token in it.  Rows past the buffer read as zero.
  const bool paged = p.pages.table != nullptr;
  const int n_rows = paged ? p.pages.pages_per_head * p.pages.page_size : p.kv_len;
  const i32x4 krsrc = buffer_rsrc_words(reinterpret_cast<const bf16_t*>(p.k) + (paged ? 0 : bi * p.ks0) + j * p.ks1,
                                        n_rows * krs);
  const i32x4 vrsrc = buffer_rsrc_words(reinterpret_cast<const bf16_t*>(p.v) + (paged ? 0 : bi * p.vs0) + j * p.vs1,
                                        n_rows * vrs);
  int arow = int(aw & 0xffffffu) * kAtom;
  if (paged && lane < na) {
    const int ps = p.pages.page_size;
    const int phys = p.pages.table[((int64_t)bi * p.Hkv + j) * p.pages.max_pages + arow / ps];
    arow = (phys >= 0 && phys < p.pages.pages_per_head) ? phys * ps + arow % ps : n_rows;
  }
  // Direct load u of a tensor writes LDS bytes 1024 u + 16 lane: stage row r,
  // physical chunk cp; it fetches the row's logical chunk cp ^ swizzle.
  int k_voff[C::kInsts], v_voff[C::kInsts];
#pragma unroll
  for (int u = 0; u < C::kInsts; ++u) {
    const int byte = u * 1024 + lane * 16;
    const int r = byte / C::kRow, cp = (byte % C::kRow) / 16;
    k_voff[u] = r * krs + (cp ^ C::swz_k(r)) * 16;
    v_voff[u] = r * vrs + (cp ^ C::swz_v(r)) * 16;
  }
  auto kst = [&](auto S) -> char* {
    constexpr int s = decltype(S)::value;
    return s == 0 ? k0 : s == 1 ? k1 : s == 2 ? k2 : k3;
  };
  auto vst = [&](auto S) -> char* {
    constexpr int s = decltype(S)::value;
    return s == 0 ? v0 : s == 1 ? v1 : s == 2 ? v2 : v3;
  };
  // issue the loads of atom `ai` of the chunk into stage S
  auto issue = [&](auto S, int ai) {
    const int row = __builtin_amdgcn_readlane(arow, ai);
    const int ko = row * krs, vo = row * vrs;
#pragma unroll
    for (int u = 0; u < C::kInsts; ++u) dma16_stream(krsrc, kst(S) + u * 1024, k_voff[u] + ko);
#pragma unroll
    for (int u = 0; u < C::kInsts; ++u) dma16_stream(vrsrc, vst(S) + u * 1024, v_voff[u] + vo);
  };

  f32x4 oacc[C::kDT];
#pragma unroll
  for (int t = 0; t < C::kDT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // l_part sums the probabilities as bf16-rounded for the P V MFMAs (the
  // normaliser of o); l_lse the same before rounding (for lse only)
  float m_run = kNegInf, l_part = 0.f, l_lse = 0.f;
  const float c2 = p.scale_log2;

  auto step = [&](auto S, int i) {
    // loads of atom i + 3 go to the stage atom i - 1 used (its reads are done)
    using SN = std::integral_constant<int, (decltype(S)::value + kDStages - 1) % kDStages>;
    if (i + kDStages - 1 < na) issue(SN{}, i + kDStages - 1);
    // wait for atom i: the loads of the atoms after it may stay in flight
    const int after = min(na - 1 - i, kDStages - 1);
    if (after >= 3) wait_vmcnt<3 * 2 * C::kInsts>();
    else if (after == 2) wait_vmcnt<2 * 2 * C::kInsts>();
    else if (after == 1) wait_vmcnt<2 * C::kInsts>();
    else wait_vmcnt<0>();
    const char* ks = kst(S);
    const char* vs = vst(S);
    const uint32_t at = uint32_t(__builtin_amdgcn_readlane(int(aw), i));
    const int tok0 = int(at & 0xffffffu) * kAtom;
    const bool sel = col < 8 && ((at >> (24 + col)) & 1u);  // head mask: bits 24 + head

    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::kDK; ++s) {
      const u32x4 a = lds16(ks, col * C::kRow + ((4 * s + qg) ^ C::swz_k(col)) * 16);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[s]),
                                                     sacc, 0, 0, 0);
    }
    float sv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[e] = (sel && tok0 + 4 * qg + e < p.kv_len) ? sacc[e] : kNegInf;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = max_xor32(max_xor16(mx));
    const float mt = mx * c2;
    const bool raise = mt > m_run + kDLazy;
    if (__builtin_expect(__ballot(raise) != 0, 0)) {
      const float m_new = raise ? mt : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 when raised from -inf
      l_part *= alpha;
      l_lse *= alpha;
#pragma unroll
      for (int t = 0; t < C::kDT; ++t) oacc[t] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], c2, -m_use));
    l_lse += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const uint32_t pk0 = pack_bf16x2(pr[0], pr[1]), pk1 = pack_bf16x2(pr[2], pr[3]);
    l_part += (bf16_lo(pk0) + bf16_hi(pk0)) + (bf16_lo(pk1) + bf16_hi(pk1));
    const v4i16 pb = __builtin_bit_cast(v4i16, uint2{pk0, pk1});
    // V^T fragments: source lane (group qg, index jj) points at V row
    // 4 qg + jj / 4, columns 16 t + 4 (jj % 4) .. +3; the lane receives
    // V[4 qg .. 4 qg + 3][16 t + jj].
    const int jj = lane & 15;
    const int vr = 4 * qg + (jj >> 2);
#pragma unroll
    for (int t = 0; t < C::kDT; ++t) {
      const int d = 16 * t + 4 * (jj & 3);
      const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(vs + vr * C::kRow + (((d >> 3) ^ C::swz_v(vr)) << 4) + ((d & 7) << 1)));
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[t], 0, 0, 0);
    }
  };

  issue(std::integral_constant<int, 0>{}, 0);
  if (na > 1) issue(std::integral_constant<int, 1>{}, 1);
  if (na > 2) issue(std::integral_constant<int, 2>{}, 2);
  for (int i = 0; i < na; i += kDStages) {
    step(std::integral_constant<int, 0>{}, i);
    if (i + 1 >= na) break;
    step(std::integral_constant<int, 1>{}, i + 1);
    if (i + 2 >= na) break;
    step(std::integral_constant<int, 2>{}, i + 2);
    if (i + 3 >= na) break;
    step(std::integral_constant<int, 3>{}, i + 3);
  }

  // partial state of this chunk: heads col < G; lane (col, qg) holds
  // d = 16 t + 4 qg .. +3
  const float l = sum_xor32(sum_xor16(l_part));
  const float lx = sum_xor32(sum_xor16(l_lse));
  if (col < p.G) {
    const int64_t r = (((int64_t)bi * p.Hkv + j) * p.n_chunks + c) * p.G + col;
#pragma unroll
    for (int t = 0; t < C::kDT; ++t) *reinterpret_cast<f32x4*>(p.part_o + r * D + 16 * t + 4 * qg) = oacc[t];
    if (qg == 0) {
      p.part_ml[r * kPartMl + 0] = m_run;
      p.part_ml[r * kPartMl + 1] = l;
      p.part_ml[r * kPartMl + 2] = lx;
    }
  }
}

// ---------------------------------------------------------------- combine
// Fixed-order merge of the chunk partials of one (batch, query head):
// o = sum_c w_c o_c / sum_c w_c l_c with w_c = 2^(m_c - max_c m_c), l_c the
// chunk's sum of the probabilities as applied to V; lse from the unrounded sums.  The
// weights of up to D chunks at a time go through LDS, so the loop over chunks
// issues independent loads.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeCombineParams p, int dtype) {
  constexpr int kW = D / 64;  // waves
  __shared__ float w_s[D + 16];  // 16 words of slack for the 16-wide unrolled reads
  __shared__ float red[kW], red2[kW];
  const int h = blockIdx.x, bi = blockIdx.y;
  const int j = h / p.G, gi = h % p.G;
  const int d = threadIdx.x, lane = d & 63, wv = d >> 6;
  const int nu = p.n_union[(int64_t)bi * p.Hkv + j];
  const int nch = (nu + p.chunk_atoms - 1) / p.chunk_atoms;
  const int64_t base = ((int64_t)bi * p.Hkv + j) * p.n_chunks;
  auto ml = [&](int c, int k) { return p.part_ml[((base + c) * p.G + gi) * kPartMl + k]; };
  float mx = kNegInf;
  for (int c = d; c < nch; c += D) mx = fmaxf(mx, ml(c, 0));
  mx = wave_max(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kW; ++i) mx = fmaxf(mx, red[i]);
  const float mu = mx == kNegInf ? 0.f : mx;
  float acc = 0.f, lp = 0.f, lq = 0.f;
  for (int c0 = 0; c0 < nch; c0 += D) {
    const int c = c0 + d;
    const float w = c < nch ? __builtin_amdgcn_exp2f(ml(c, 0) - mu) : 0.f;
    lp += c < nch ? w * ml(c, 1) : 0.f;
    lq += c < nch ? w * ml(c, 2) : 0.f;
    __syncthreads();
    w_s[d] = w;
    __syncthreads();
    const int cn = min(D, nch - c0);
    const float* po = p.part_o + ((base + c0) * p.G + gi) * D + d;
    const int64_t cs = (int64_t)p.G * D;  // chunk stride
    // 16 independent loads per round trip; chunks past cn read chunk 0 with weight 0
    for (int u0 = 0; u0 < cn; u0 += 16) {
      float a[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) a[u] = po[(u0 + u < cn ? u0 + u : 0) * cs];
#pragma unroll
      for (int u = 0; u < 16; ++u) acc = fmaf(a[u], u0 + u < cn ? w_s[u0 + u] : 0.f, acc);
    }
  }
  lp = wave_sum(lp);
  lq = wave_sum(lq);
  __syncthreads();
  if (lane == 0) {
    red[wv] = lp;
    red2[wv] = lq;
  }
  __syncthreads();
  float l = 0.f, lx = 0.f;
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    l += red[i];
    lx += red2[i];
  }
  const float o = l > 0.f ? acc / l : 0.f;
  const int64_t oi = bi * p.os0 + h * p.os1 + d;
  if (p.out_f32 || dtype == 1) reinterpret_cast<float*>(p.o)[oi] = o;
  else reinterpret_cast<bf16_t*>(p.o)[oi] = bf16_t(pack_bf16x2(o, 0.f) & 0xffffu);
  if (p.lse && d == 0) p.lse[(int64_t)bi * p.Hq + h] = lx > 0.f ? (mx + __log2f(lx)) * kLn2 : kNegInf;
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
    if (p.G > 8 || p.chunk_atoms > 64) return hipErrorInvalidValue;
    if (D == 128) hipLaunchKernelGGL(decode_attn_mfma_kernel<128>, grid, dim3(64), 0, stream, p);
    else if (D == 64) hipLaunchKernelGGL(decode_attn_mfma_kernel<64>, grid, dim3(64), 0, stream, p);
    else return hipErrorInvalidValue;
  } else {
    if (p.pages.table) return hipErrorInvalidValue;  // paged caches: bf16 only
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
