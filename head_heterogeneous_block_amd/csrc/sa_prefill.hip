// Block-sparse causal prefill attention for gfx950 (CDNA4, wave64).
//
// Exact softmax attention of every query row over the keys of the key blocks
// its (head, query block) tile selected, flash-style (online softmax, one pass
// over the gathered blocks).  Per-head top-k sparse attention: "S-HPLB:
// Efficient LLM Attention Serving via Sparsity-Aware Head Parallelism Load
// Balance", Italian summary §1-2 / Chinese summary §1-2.  The persistent
// workgroups walk the bins of a greedy longest-load-first schedule (same pages,
// §2.B / §2.2) so large-budget heads do not leave compute units idle at the
// tail.
//
// Work decomposition
//   tile      = (batch b, query head h, query block m): B query rows.
//   workgroup = W waves; wave w owns query rows [w*B/W, (w+1)*B/W) of the tile.
//   step      = 64 keys of one selected key block (B/64 steps per block).
//   K and V of a step are gathered from HBM through the block-index table with
//   buffer loads (the (batch, KV head) slice is the buffer, so rows past the
//   end of the sequence read as zero), double-buffered in LDS (K row-major, V
//   transposed) and XOR-swizzled so that the 16-byte LDS reads of the MFMA
//   operands do not conflict.  While step s is computed from one stage, step
//   s+1 is fetched: K first, V once Q K^T of step s is done.
//
// Math per step and wave (bf16 path):
//   S^T[key][q] = K Q^T    v_mfma_f32_32x32x16_bf16, A = K rows (LDS),
//                          B = Q^T (registers, loaded once per tile).
//   With S transposed every lane column is one query, so the row max and row
//   sum of the online softmax are in-lane plus one exchange between the two
//   half-waves.
//   O^T[d][q] += V^T P^T   A = V^T rows (LDS), B = P^T straight from the S^T
//                          accumulators.  For that, key rows are stored in LDS
//                          with bits 2 and 3 of the key index swapped: the
//                          accumulator element i of a lane then holds key
//                          16*(i/8) + 8*half + i%8, i.e. 8 consecutive keys per
//                          16-key chunk, which is the B-operand layout.
//   fp32 path: v_mfma_f32_32x32x2f32 with the same layouts, P kept in fp32.
// Softmax: scores stay unscaled; exp2(s*c - m) with c = scale*log2(e) is one
// FMA and one v_exp_f32.  The running max m is only raised when a new score
// exceeds it by more than 2^kLazy (then O and l are rescaled, decided per wave),
// so p <= 2^kLazy; l and O use the same m, so the result is unchanged.

#include "sa_device.hpp"
#include "sa_kernels.hpp"

namespace sa {

namespace {

constexpr int kKS = 64;        // keys per step
constexpr float kLazy = 8.f;   // log2 headroom before the running max is raised

// swap bits 2 and 3 of a key index (an involution)
__device__ __forceinline__ int perm_key(int k) { return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1); }

// 16-byte chunk swizzles
__device__ __forceinline__ int swz_k(int row, int chunk) { return chunk ^ (row & 7); }
__device__ __forceinline__ int swz_v(int drow, int chunk) { return chunk ^ ((drow + (drow >> 3)) & 7); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 lds16(const char* base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(base + byte_off);
}
template <int BYTES>
__device__ __forceinline__ void sts(char* base, int byte_off, const uint32_t* w) {
  if constexpr (BYTES == 16) {
    *reinterpret_cast<u32x4*>(base + byte_off) = u32x4{w[0], w[1], w[2], w[3]};
  } else if constexpr (BYTES == 8) {
    *reinterpret_cast<uint2*>(base + byte_off) = uint2{w[0], w[1]};
  } else {
    *reinterpret_cast<uint32_t*>(base + byte_off) = w[0];
  }
}

template <typename T, int D, int B, int W>
struct Cfg {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kThreads = 64 * W;
  static constexpr int kE16 = 16 / int(sizeof(T));  // elements per 16 bytes
  static constexpr int kNSub = B / kKS;             // steps per key block
  static constexpr int kQPW = B / W;                // queries per wave
  static constexpr int kQT = kQPW / 32;             // 32-query MFMA column tiles per wave
  static constexpr int kDT = D / 32;                // 32-row d tiles of O^T
  static constexpr int kKRowBytes = D * int(sizeof(T));
  static constexpr int kKChunks = kKRowBytes / 16;  // 16-byte chunks per K row
  static constexpr int kVRowBytes = kKS * int(sizeof(T));
  static constexpr int kKBytes = kKS * kKRowBytes;
  static constexpr int kVBytes = D * kVRowBytes;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kKLoads = kKS * kKChunks / kThreads;  // 16-byte K loads per thread
  static constexpr int kKRowsPerLoad = kThreads / kKChunks;
  // V transpose unit: kVK keys x kE16 d (one 16-byte load per key row),
  // written as kE16 transposed runs of kVK elements
  static constexpr int kVKWant = kKS * D / (kE16 * kThreads);
  static constexpr int kVK = kVKWant > kE16 ? kE16 : (kVKWant < 2 ? 2 : kVKWant);
  static constexpr int kVUnits = (kKS / kVK) * (D / kE16);
  static constexpr int kVUnitsPerThread = (kVUnits + kThreads - 1) / kThreads;
  static constexpr int kVWrite = kVK * int(sizeof(T));  // bytes per transposed run
  static constexpr int kDG = D / (2 * kE16);            // Q K^T k-groups (16 B per lane)
  static_assert(kQT >= 1, "at least 32 queries per wave");
  static_assert(kKLoads * kThreads == kKS * kKChunks, "K loads must divide evenly");
};

struct Step {
  int valid;
  int item;  // index into the bin's item list
  int tile;
  int j;     // position in the tile's block list
  int hs;    // step within the key block
  int cnt;   // blocks of this tile
  int n;     // key block index
};

__device__ __forceinline__ int tile_of(const PrefillParams& p, int item) {
  return p.items_by_bin ? p.items_by_bin[item] : item;
}

// key block j of a tile, or -1 if the table holds something outside 0..m
__device__ __forceinline__ int block_at(const PrefillParams& p, int tile, int j) {
  const int n = wave_uniform(p.block_idx[(int64_t)tile * p.kmax + j]);
  return (n >= 0 && n <= tile % p.NB) ? n : -1;
}

// first step at or after (item it, block j) whose block entry is valid
__device__ __forceinline__ void seek(const PrefillParams& p, int it, int j, int it_end, Step& s) {
  s.valid = 0;
  for (; it < it_end; ++it, j = 0) {
    const int tile = wave_uniform(tile_of(p, it));
    if (tile < 0 || tile >= p.n_tiles) continue;
    const int cnt = min(wave_uniform(p.block_cnt[tile]), p.kmax);
    for (; j < cnt; ++j) {
      const int n = block_at(p, tile, j);
      if (n >= 0) {
        s.valid = 1;
        s.item = it;
        s.tile = tile;
        s.j = j;
        s.hs = 0;
        s.cnt = cnt;
        s.n = n;
        return;
      }
    }
  }
}

template <int NSUB>
__device__ __forceinline__ void advance(const PrefillParams& p, int it_end, Step& s) {
  if (s.hs + 1 < NSUB) {
    s.hs += 1;
    return;
  }
  seek(p, s.item, s.j + 1, it_end, s);
}

template <typename T, int D, int B, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W == 4 ? 2 : 1, W == 4 ? 2 : 1))) void prefill_kernel(PrefillParams p) {
  using C = Cfg<T, D, B, W>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // MFMA column (query) / A-row (key, d) index
  const int half = lane >> 5;  // MFMA k-half

  int it_beg, it_end;
  if (p.bin_offsets) {
    it_beg = p.bin_offsets[blockIdx.x];
    it_end = p.bin_offsets[blockIdx.x + 1];
  } else {
    it_beg = blockIdx.x;
    it_end = (int)blockIdx.x < p.n_tiles ? (int)blockIdx.x + 1 : (int)blockIdx.x;
  }
  const int NB = p.NB;
  const int S = p.S;
  const float c2 = p.scale_log2;

  // ---------------------------------------------------------------- loads
  u32x4 kreg[C::kKLoads];
  u32x4 vreg[C::kVUnitsPerThread][C::kVK];
  const int krs = int(p.ks2 * (int64_t)sizeof(T));
  const int vrs = int(p.vs2 * (int64_t)sizeof(T));
  const int k_voff = (tid / C::kKChunks) * krs + (tid % C::kKChunks) * 16;

  auto slice = [&](int tile, const void* base, int64_t s0, int64_t s1, int rs) {
    const int bi = tile / (p.Hq * NB);
    const int h = (tile / NB) % p.Hq;
    const char* b = reinterpret_cast<const char*>(base) + (bi * s0 + (h / p.G) * s1) * (int64_t)sizeof(T);
    return __builtin_amdgcn_make_buffer_rsrc((void*)b, (short)0, S * rs, 0x00020000);
  };
  auto load_k = [&](const Step& s) {
    const auto rk = slice(s.tile, p.k, p.ks0, p.ks1, krs);
    const int key0 = s.n * B + s.hs * kKS;
#pragma unroll
    for (int i = 0; i < C::kKLoads; ++i)
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_voff, (key0 + i * C::kKRowsPerLoad) * krs, 0);
  };
  auto load_v = [&](const Step& s) {
    const auto rv = slice(s.tile, p.v, p.vs0, p.vs1, vrs);
    const int key0 = s.n * B + s.hs * kKS;
#pragma unroll
    for (int u = 0; u < C::kVUnitsPerThread; ++u) {
      const int unit = u * C::kThreads + tid;
      if (unit < C::kVUnits) {
        const int dc = unit % (D / C::kE16), kg = unit / (D / C::kE16);
        const int voff = kg * C::kVK * vrs + dc * 16;
#pragma unroll
        for (int e = 0; e < C::kVK; ++e)
          vreg[u][e] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, (key0 + e) * vrs, 0);
      }
    }
  };
  auto store_k = [&](int stage) {
    char* ks = smem + stage * C::kStage;
#pragma unroll
    for (int i = 0; i < C::kKLoads; ++i) {
      const int flat = i * C::kThreads + tid;
      const int r = flat / C::kKChunks, c = flat % C::kKChunks;
      const int lr = perm_key(r);
      *reinterpret_cast<u32x4*>(ks + lr * C::kKRowBytes + swz_k(lr, c) * 16) = kreg[i];
    }
  };
  auto store_v = [&](int stage) {
    char* vs = smem + stage * C::kStage + C::kKBytes;
#pragma unroll
    for (int u = 0; u < C::kVUnitsPerThread; ++u) {
      const int unit = u * C::kThreads + tid;
      if (unit < C::kVUnits) {
        const int dc = unit % (D / C::kE16), kg = unit / (D / C::kE16);
        const int kbyte = kg * C::kVWrite;  // byte offset of the run within a V^T row
#pragma unroll
        for (int e = 0; e < C::kE16; ++e) {
          uint32_t w[4];
          if constexpr (C::kBf16) {
            // column e (d = 8*dc + e) of the kVK key rows, packed two keys per word
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int t = 0; t < C::kVK / 2; ++t)
              w[t] = __builtin_amdgcn_perm(vreg[u][2 * t + 1][e >> 1], vreg[u][2 * t][e >> 1], sel);
          } else {
#pragma unroll
            for (int t = 0; t < C::kVK; ++t) w[t] = vreg[u][t][e];
          }
          const int drow = dc * C::kE16 + e;
          sts<C::kVWrite>(vs, drow * C::kVRowBytes + swz_v(drow, kbyte >> 4) * 16 + (kbyte & 15), w);
        }
      }
    }
  };

  // ---------------------------------------------------------------- tile state
  u32x4 qf[C::kQT][C::kDG];  // Q^T fragments
  f32x16 oacc[C::kDT][C::kQT];
  float m_run[C::kQT], l_run[C::kQT];

  auto start_tile = [&](int tile) {
    const int bi = tile / (p.Hq * NB);
    const int h = (tile / NB) % p.Hq;
    const int m = tile % NB;
    const char* qb = reinterpret_cast<const char*>(p.q) + (bi * p.qs0 + h * p.qs1) * (int64_t)sizeof(T);
#pragma unroll
    for (int qt = 0; qt < C::kQT; ++qt) {
      const int qrow = m * B + wave * C::kQPW + qt * 32 + col;
      const char* rp = qb + (int64_t)qrow * p.qs2 * (int64_t)sizeof(T);
#pragma unroll
      for (int dg = 0; dg < C::kDG; ++dg) {
        // bf16: lane half g holds d = 16*dg + 8*g .. +7; fp32: d = 8*dg + 4*g .. +3
        const int d0 = dg * 2 * C::kE16 + half * C::kE16;
        qf[qt][dg] = qrow < S ? ldg16(rp + d0 * (int)sizeof(T)) : u32x4{0u, 0u, 0u, 0u};
      }
      m_run[qt] = kNegInf;
      l_run[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) oacc[dt][qt] = f32x16{};
    }
  };

  auto finish_tile = [&](int tile) {
    const int bi = tile / (p.Hq * NB);
    const int h = (tile / NB) % p.Hq;
    const int m = tile % NB;
#pragma unroll
    for (int qt = 0; qt < C::kQT; ++qt) {
      const float l = l_run[qt] + __shfl_xor(l_run[qt], 32, 64);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int qrow = m * B + wave * C::kQPW + qt * 32 + col;
      if (qrow < S) {
        const int64_t orow = bi * p.os0 + h * p.os1 + (int64_t)qrow * p.os2;
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d = dt * 32 + r4 * 8 + half * 4;
            const float o0 = oacc[dt][qt][r4 * 4 + 0] * inv, o1 = oacc[dt][qt][r4 * 4 + 1] * inv;
            const float o2 = oacc[dt][qt][r4 * 4 + 2] * inv, o3 = oacc[dt][qt][r4 * 4 + 3] * inv;
            if (C::kBf16 && !p.out_f32) {
              uint2 w;
              w.x = pack_bf16x2(o0, o1);
              w.y = pack_bf16x2(o2, o3);
              *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(p.o) + orow + d) = w;
            } else {
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + orow + d) = f32x4{o0, o1, o2, o3};
            }
          }
        }
        if (p.lse && half == 0)
          p.lse[((int64_t)bi * p.Hq + h) * S + qrow] = l > 0.f ? (m_run[qt] + __log2f(l)) * kLn2 : kNegInf;
      }
    }
  };

  // ---------------------------------------------------------------- one step
  auto compute_step = [&](const Step& s, int stage, const Step& nx) {
    const int m = s.tile % NB;
    const int n = s.n;
    const int key0 = s.hs * kKS;      // first key of the step within block n
    const int q_lo = wave * C::kQPW;  // first query of the wave within block m
    // the whole step lies above the causal diagonal for this wave
    if (n == m && key0 > q_lo + C::kQPW - 1) {
      if (nx.valid) {
        store_k(stage ^ 1);
        load_v(nx);
      }
      return;
    }
    const bool diag = (n == m) && (key0 + kKS - 1 > q_lo);
    const bool tail = (n * B + key0 + kKS > S);
    const char* ks = smem + stage * C::kStage;
    const char* vs = ks + C::kKBytes;

    f32x16 sacc[2][C::kQT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < C::kQT; ++qt) sacc[kt][qt] = f32x16{};

    // ---- S^T = K Q^T
#pragma unroll
    for (int dg = 0; dg < C::kDG; ++dg) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int r = kt * 32 + col;
        const u32x4 a = lds16(ks, r * C::kKRowBytes + swz_k(r, dg * 2 + half) * 16);
#pragma unroll
        for (int qt = 0; qt < C::kQT; ++qt) {
          if constexpr (C::kBf16) {
            sacc[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[qt][dg]), sacc[kt][qt], 0, 0, 0);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sacc[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(qf[qt][dg][e]),
                                                                  sacc[kt][qt], 0, 0, 0);
          }
        }
      }
    }

    // K of the next step goes to the other stage now; V of the next step is
    // fetched while the softmax and P V run
    if (nx.valid) {
      store_k(stage ^ 1);
      load_v(nx);
    }

    // ---- online softmax in the log2 domain
#pragma unroll
    for (int qt = 0; qt < C::kQT; ++qt) {
      if (diag || tail) {
        const int q_in_blk = q_lo + qt * 32 + col;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kl = key0 + kt * 32 + (i >> 3) * 16 + half * 8 + (i & 7);
            const bool masked = (diag && kl > q_in_blk) || (tail && n * B + kl >= S);
            if (masked) sacc[kt][qt][i] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][qt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
      // raise the running max only when a score gets 2^kLazy above it
      const bool raise = mx > m_run[qt] + kLazy;
      if (__ballot(raise) != 0) {
        const float m_new = raise ? mx : m_run[qt];
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run[qt] - m_new) : 1.f;  // 0 when m_run = -inf
        l_run[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) oacc[dt][qt] *= alpha;
        m_run[qt] = m_new;
      }
      const float m_use = m_run[qt] == kNegInf ? 0.f : m_run[qt];
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kt][qt][i], c2, -m_use));
          sacc[kt][qt][i] = pv;
          psum += pv;
        }
      l_run[qt] += psum;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kt = kc >> 1, c = kc & 1;
      if constexpr (C::kBf16) {
        u32x4 pf[C::kQT];
#pragma unroll
        for (int qt = 0; qt < C::kQT; ++qt)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            pf[qt][w] = pack_bf16x2(sacc[kt][qt][8 * c + 2 * w], sacc[kt][qt][8 * c + 2 * w + 1]);
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) {
          const int drow = dt * 32 + col;
          const u32x4 a = lds16(vs, drow * C::kVRowBytes + swz_v(drow, kc * 2 + half) * 16);
#pragma unroll
          for (int qt = 0; qt < C::kQT; ++qt)
            oacc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pf[qt]), oacc[dt][qt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) {
          const int drow = dt * 32 + col;
          // keys 16*kc + 8*half .. +7: two 16-byte chunks
          const u32x4 a0 = lds16(vs, drow * C::kVRowBytes + swz_v(drow, kc * 4 + half * 2) * 16);
          const u32x4 a1 = lds16(vs, drow * C::kVRowBytes + swz_v(drow, kc * 4 + half * 2 + 1) * 16);
#pragma unroll
          for (int qt = 0; qt < C::kQT; ++qt)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              oacc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(e < 4 ? a0[e & 3] : a1[e & 3]),
                                                                  sacc[kt][qt][8 * c + e], oacc[dt][qt], 0, 0, 0);
        }
      }
    }
  };

  // ---------------------------------------------------------------- walk
  Step cur, nxt;
  seek(p, it_beg, 0, it_end, cur);
  if (!cur.valid) return;
  load_k(cur);
  load_v(cur);
  store_k(0);
  store_v(0);
  __syncthreads();
  nxt = cur;
  advance<C::kNSub>(p, it_end, nxt);
  start_tile(cur.tile);
  int stage = 0;
  while (true) {
    if (nxt.valid) load_k(nxt);
    compute_step(cur, stage, nxt);
    const bool tile_done = !nxt.valid || nxt.tile != cur.tile || nxt.item != cur.item;
    if (tile_done) finish_tile(cur.tile);
    if (nxt.valid) store_v(stage ^ 1);
    __syncthreads();
    if (!nxt.valid) break;
    if (tile_done) start_tile(nxt.tile);
    cur = nxt;
    advance<C::kNSub>(p, it_end, nxt);
    stage ^= 1;
  }
}

template <typename T, int D, int B, int W>
hipError_t launch_t(const PrefillParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<T, D, B, W>), dim3(grid), dim3(64 * W), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int D, int B, int waves, int grid, hipStream_t stream) {
  if (dtype == 0) {
    if (waves == 2) {
      if (D == 128 && B == 128) return launch_t<bf16_t, 128, 128, 2>(p, grid, stream);
      if (D == 128 && B == 64) return launch_t<bf16_t, 128, 64, 2>(p, grid, stream);
      if (D == 64 && B == 128) return launch_t<bf16_t, 64, 128, 2>(p, grid, stream);
      if (D == 64 && B == 64) return launch_t<bf16_t, 64, 64, 2>(p, grid, stream);
    } else if (waves == 4) {
      if (D == 128 && B == 128) return launch_t<bf16_t, 128, 128, 4>(p, grid, stream);
      if (D == 64 && B == 128) return launch_t<bf16_t, 64, 128, 4>(p, grid, stream);
    }
  } else if (waves == 2) {
    if (D == 128 && B == 64) return launch_t<float, 128, 64, 2>(p, grid, stream);
    if (D == 64 && B == 64) return launch_t<float, 64, 64, 2>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
