// Block selection kernels for gfx950: mean pooling, block scores and the exact
// per-row top-k with forced sink/local blocks.
//
//  * pooling: the Index step of "Unifying Sparse Attention with Hierarchical
//    Memory for Scalable Long-Context LLM Serving" (Spin), Spanish summary
//    §2.A, at block granularity ("Fluxion", Italian summary, Intuizioni
//    Chiave 2): the mean of the rows of every block, accumulated in fp32.
//  * scoring + top-k: the Select step (same passage) with per-head budgets
//    ("S-HPLB ...", Italian summary §2.A, Chinese summary §2.1) and a top-k
//    token budget per head (same pages §1).
//
// Top-k is exact: scores become order-preserving 32-bit keys; the k'-th largest
// key is found by a byte-wise radix select over block-wide histograms; blocks
// with a larger key, and the first (lowest-index) ties, are kept.  Candidates
// are laid out in index order over the threads, so the output comes out
// ascending with no sort.

#include <type_traits>

#include "sa_device.hpp"
#include "sa_kernels.hpp"

namespace sa {

namespace {

// ---------------------------------------------------------------- pooling
// One workgroup (256 threads) pools `blocks_per_wg` consecutive blocks of one
// (batch, head).  Each thread owns one 16-byte column chunk and a strided set
// of rows; row groups are combined through LDS.
template <typename T, int D, bool kNorm>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  constexpr int kE = 16 / int(sizeof(T));  // elements per chunk
  constexpr int kCh = D / kE;              // chunks per row
  constexpr int kRG = 256 / kCh;           // row groups
  static_assert(kCh == 8 || kCh == 16 || kCh == 32, "a row's chunks are 8, 16 or 32 consecutive lanes");
  __shared__ float part[kRG][D + 1];
  __shared__ float nrm[kRG];
  const int tid = threadIdx.x;
  const int ch = tid % kCh, rg = tid / kCh;
  const int h = blockIdx.y, bi = blockIdx.z;
  const bool paged = p.pages.table != nullptr;
  const char* base = reinterpret_cast<const char*>(p.x) + ((paged ? 0 : bi * p.s0) + h * p.s1) * (int64_t)sizeof(T);
  const int64_t rs = p.s2 * (int64_t)sizeof(T);
  for (int bb = 0; bb < p.blocks_per_wg; ++bb) {
    const int n = blockIdx.x * p.blocks_per_wg + bb;
    if (n >= p.nb) break;
    int lo = n * p.g;
    const int cnt = min(p.g, p.T - lo);
    if (paged) {
      // the block lies in one page (g divides the page size): its first row in
      // the pool; rows of an out-of-range page entry are not read
      const int ps = p.pages.page_size;
      const int phys = p.pages.table[((int64_t)bi * p.heads + h) * p.pages.max_pages + lo / ps];
      if (phys < 0 || phys >= p.pages.pages_per_head) {
        for (int d = tid; d < D; d += 256) p.out[(((int64_t)bi * p.heads + h) * p.nb + n) * D + d] = 0.f;
        continue;
      }
      lo = phys * ps + lo % ps;
    }
    float acc[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = 0.f;
    float n2max = 0.f;  // kNorm: largest squared norm among this row group's rows
    // eight rows' loads in flight per thread, then summed in row order (rows
    // past the block end read as zeros, which leave the sums unchanged)
    for (int r0 = rg; r0 < cnt; r0 += 8 * kRG) {
      u32x4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + u * kRG;
        // read once: non-temporal, so the rows are not kept in the caches
        w[u] = r < cnt ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (int64_t)(lo + r) * rs + ch * 16))
                       : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += bf16_lo(w[u][e]);
            acc[2 * e + 1] += bf16_hi(w[u][e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[u][e]);
        }
      }
      if constexpr (kNorm) {
        // squared norm of each of the eight rows: this lane's chunk, then the
        // row's kCh consecutive lanes
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          // plain FMAs: ROCm 7.2's compiler folds chains of v_dot2 over
          // elements of a vector wrongly (some pairs read twice)
          float q2 = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (sizeof(T) == 2) {
              const float lo = bf16_lo(w[u][e]), hi = bf16_hi(w[u][e]);
              q2 = fmaf(lo, lo, fmaf(hi, hi, q2));
            } else {
              const float x = __uint_as_float(w[u][e]);
              q2 = fmaf(x, x, q2);
            }
          }
          if constexpr (kCh == 8) q2 = sum8(q2);
          else q2 = row_sum16(q2);
          if constexpr (kCh == 32) q2 += __shfl_xor(q2, 16);
          n2max = fmaxf(n2max, q2);
        }
      }
    }
    if constexpr (kNorm) {
      if (ch == 0) nrm[rg] = n2max;
    }
#pragma unroll
    for (int e = 0; e < kE; ++e) part[rg][ch * kE + e] = acc[e];
    __syncthreads();
    for (int d = tid; d < D; d += 256) {
      float s = 0.f;
#pragma unroll 8
      for (int r = 0; r < kRG; ++r) s += part[r][d];
      p.out[(((int64_t)bi * p.heads + h) * p.nb + n) * D + d] = s / float(cnt);
    }
    if constexpr (kNorm) {
      if (tid == 0) {
        float m2 = 0.f;
        for (int r = 0; r < kRG; ++r) m2 = fmaxf(m2, nrm[r]);
        p.norm_max[((int64_t)bi * p.heads + h) * p.nb + n] = __builtin_sqrtf(m2);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- prefill selection
// One kernel per selection: pooling of the query blocks, their scores against
// the pooled keys, and the per-row top-k, with nothing between the steps
// leaving the chip (the scores of a workgroup's rows live in LDS).
//
// Workgroup = up to R consecutive query blocks m0 .. m0+R-1 of one (sequence,
// query head) (R = 16 for up to 1024 blocks, fewer for longer sequences so the
// rows fit in LDS); the workgroups of the last query blocks, which score the
// most keys, start first.
//   1. pool: the R blocks' rows of Q, summed in fp32 (16-byte non-temporal
//      loads, two blocks' loads in flight per thread), divided by the row
//      count: the block means Qbar, in LDS;
//   2. score: S[r][n] = scale * <Qbar[r], Kbar[n]> for n < m0 + R on the fp32
//      MFMA pipe (v_mfma_f32_16x16x4f32: A = the 16 rows of Qbar, held in
//      registers; B = 16 pooled keys read from L2; lane group g of the wave
//      takes channels [g D/4, (g+1) D/4), so each MFMA consumes 4 channels and
//      D/4 of them cover the dot product).  fp32 keeps the scores exact enough
//      for the 1e-4 relative gaps the selection is checked against;
//   3. top-k: wave w takes rows w, w+4, ...: the exact radix select of the
//      key bytes (below), reading the row's keys from LDS.
// Exact top-k of one row of scores by one wave (the Select step's per-row
// budget): forced candidates ([0, ns) and [nl_lo, n_cand)) are kept, and kk of
// the others are picked, the largest keys (order-preserving maps of the
// scores), ties to the lowest index.  Lane l owns candidates [l cpt, (l+1) cpt).
// The kk-th largest key is found by a radix select over the bytes of
// rel = key - min + 1 (0 = not rankable), from the top set bit of the range
// down, with a 256-bin LDS histogram per pass (hw: two of them, alternating);
// one scan of the per-lane counts then places the kept candidates in ascending
// index order.  With kReg, cpt = kC and every rel stays in a register;
// otherwise cpt = ceil(n_cand / 64) and each pass reads the row again from LDS.
template <int kC, bool kReg>
__device__ __forceinline__ void topk_row_wave(const float* srow, int n_cand, int k, int kk, int ns, int nl_lo,
                                              int32_t* out, int lane, uint32_t* hw) {
  const int cpt = kReg ? kC : (n_cand + 63) >> 6;
  const int n0 = lane * cpt;
  uint32_t regs[kReg ? kC : 1];
  auto key_of = [&](int c) -> uint32_t {
    const int n = n0 + c;
    const int nn = min(n, n_cand - 1);  // reads stay in the row
    const float v = srow[nn + (nn >> 5)];
    return (n < n_cand && n >= ns && n < nl_lo) ? ordered_key(v) : 0u;
  };
  uint32_t kmin = 0xffffffffu, kmx = 0u;
  if constexpr (kReg) {
#pragma unroll
    for (int c = 0; c < kC; ++c) regs[c] = key_of(c);  // every read issued before any is used
  }
#pragma unroll(kReg ? kC : 4)
  for (int c = 0; c < cpt; ++c) {
    const uint32_t key = kReg ? regs[c] : key_of(c);
    if (key != 0u) {
      kmin = min(kmin, key);
      kmx = max(kmx, key);
    }
  }
  kmin = wave_umin(kmin);
  kmx = wave_umax(kmx);
  if constexpr (kReg) {
#pragma unroll
    for (int c = 0; c < kC; ++c) regs[c] = regs[c] != 0u ? regs[c] - kmin + 1u : 0u;
  }
  auto rel_of = [&](int c) -> uint32_t {
    if constexpr (kReg) return regs[c];
    const uint32_t key = key_of(c);
    return key != 0u ? key - kmin + 1u : 0u;
  };
  const uint32_t range = kmx - kmin + 1u;  // >= 1: more than kk >= 1 rankable keys exist
  const int bits = 32 - __clz(range);
  uint32_t prefix = 0, pmask = 0, need = uint32_t(kk);
  uint32_t thr = 0, ties_wanted = 0;
  int width = bits < 8 ? bits : 8;
  int shift = bits - width;
#pragma unroll
  for (int u = 0; u < 4; ++u) hw[4 * lane + u] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll 1
  for (int pass = 0;; ++pass) {
    uint32_t* const hh = hw + (pass & 1) * 256;
    const uint32_t dmask = (1u << width) - 1u;
#pragma unroll(kReg ? kC : 4)
    for (int c = 0; c < cpt; ++c) {
      const uint32_t rel = rel_of(c);
      if (rel != 0u && (rel & pmask) == prefix) atomicAdd(&hh[(rel >> shift) & dmask], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // the digit whose bin holds the need-th largest key: lane l scans bins
    // 255 - 4l .. 252 - 4l (digits in descending order)
    uint32_t hc[4], loc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      hc[u] = hh[255 - (4 * lane + u)];
      loc += hc[u];
    }
    uint32_t above = wave_scan_incl(loc) - loc;
    int hit = -1;
    uint32_t h_rem = 0, h_bin = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (hit < 0 && above < need && above + hc[u] >= need) {
        hit = u;
        h_rem = need - above;
        h_bin = hc[u];
      }
      above += hc[u];
    }
    const int src = int(__builtin_ctzll(__ballot(hit >= 0)));
    const int hu = __builtin_amdgcn_readlane(hit, src);
    const uint32_t digit = 255u - uint32_t(4 * src + hu);
    const uint32_t rem = uint32_t(__builtin_amdgcn_readlane(int(h_rem), src));
    const uint32_t bin = uint32_t(__builtin_amdgcn_readlane(int(h_bin), src));
    uint32_t* const hn = hw + ((pass + 1) & 1) * 256;  // cleared for the next pass
#pragma unroll
    for (int u = 0; u < 4; ++u) hn[4 * lane + u] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    prefix |= digit << shift;
    pmask |= dmask << shift;
    need = rem;
    if (rem == bin && prefix != 0u) {
      thr = prefix - 1u;  // every key of this bin is kept: threshold just below it
      ties_wanted = 0;
      break;
    }
    if (shift == 0) {
      thr = prefix;
      ties_wanted = rem;
      break;
    }
    width = shift < 8 ? shift : 8;
    shift -= width;
  }
  // kept: forced, rel > thr, and the ties_wanted lowest-index rel == thr; one
  // scan of the packed counts (ties << 16 | kept) gives each lane its first
  // output position and the ties at lower indices
  uint32_t n_tie = 0, n_gt = 0;
#pragma unroll(kReg ? kC : 4)
  for (int c = 0; c < cpt; ++c) {
    const int n = n0 + c;
    const uint32_t rel = rel_of(c);
    if (n < n_cand) {
      if (rel == 0u || rel > thr) ++n_gt;  // forced (rel 0), or above the threshold
      else if (rel == thr) ++n_tie;
    }
  }
  const uint32_t packed = (n_tie << 16) | n_gt;
  const uint32_t before = wave_scan_incl(packed) - packed;
  // (written without a guarded subtraction; see the decode top-k below)
  const uint32_t taken_before = min(before >> 16, ties_wanted);
  uint32_t ties_left = min(n_tie, ties_wanted - taken_before);
  uint32_t pos = (before & 0xffffu) + taken_before;
#pragma unroll(kReg ? kC : 4)
  for (int c = 0; c < cpt; ++c) {
    const int n = n0 + c;
    const uint32_t rel = rel_of(c);
    bool take = false;
    if (n < n_cand) {
      take = rel == 0u || rel > thr;
      if (!take && rel == thr && ties_left > 0u) {
        take = true;
        --ties_left;
      }
    }
    if (take && pos < uint32_t(k)) out[pos++] = n;
  }
}

template <typename T, int D, int B>
__global__ __launch_bounds__(256, 2) void select_prefill_kernel(PrefillSelectParams p) {
  __shared__ float sarea[kSelFloats];
  __shared__ uint32_t hist[4][2][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int BH = int(gridDim.x) / p.n_mg;
  const int mg = p.n_mg - 1 - int(blockIdx.x) / BH;  // heaviest rows first
  const int bh = int(blockIdx.x) % BH;
  const int bi = bh / p.Hq, h = bh % p.Hq;
  const int bkv = bi * (p.Hq / p.G) + h / p.G;
  const int m0 = mg * p.R;
  const int R = min(p.R, p.NB - m0);

  // the first two key tiles of this wave's scoring load while the queries pool
  constexpr int kJ = D / 4;  // MFMAs per 16 x 16 tile
  const int ci = lane & 15, kg = lane >> 4;
  const int ncols = m0 + R;  // score columns 0 .. m0+R-1
  const int ntiles = (ncols + 15) >> 4;
  const float* kb = p.kp + int64_t(bkv) * p.NB * D + kg * kJ;
  auto load_b = [&](int t, float (&b)[kJ]) {
    const int n = t * 16 + ci;
    if (t < ntiles && n < p.NB) {
#pragma unroll
      for (int j = 0; j < kJ; j += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(kb + int64_t(n) * D + j);
        b[j] = v[0];
        b[j + 1] = v[1];
        b[j + 2] = v[2];
        b[j + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kJ; ++j) b[j] = 0.f;
    }
  };
  float b0[kJ], b1[kJ];
  load_b(wave, b0);
  load_b(wave + 4, b1);

  // ---- 1. pool
  constexpr int kE = 16 / int(sizeof(T));  // elements per 16-byte chunk
  constexpr int kCh = D / kE;              // chunks per row
  constexpr int kRG = 256 / kCh;           // row groups
  constexpr int kRPT = B / kRG;            // rows per thread per block
  static_assert(kRPT >= 1 && B % kRG == 0, "row split");
  static_assert(2 * kRG * (D + 1) + kSelRows * D <= kSelFloats, "pool area");
  float* part = sarea;                      // [2][kRG][D + 1]
  float* qbar = sarea + 2 * kRG * (D + 1);  // [kSelRows][D]
  {
    const int ch = tid % kCh, rg = tid / kCh;
    const char* qb = static_cast<const char*>(p.q) + (bi * p.qs0 + h * p.qs1) * int64_t(sizeof(T));
    const int64_t rs = p.qs2 * int64_t(sizeof(T));
    for (int r0 = 0; r0 < R; r0 += 2) {
      int cnt[2];
      u32x4 w[2][kRPT];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int lo = (m0 + r0 + u) * B;
        cnt[u] = r0 + u < R ? min(B, p.S - lo) : 0;
#pragma unroll
        for (int i = 0; i < kRPT; ++i) {
          const int row = rg + i * kRG;
          w[u][i] = row < cnt[u] ? __builtin_nontemporal_load(
                                       reinterpret_cast<const u32x4*>(qb + int64_t(lo + row) * rs + ch * 16))
                                 : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float acc[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < kRPT; ++i) {
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[2 * e] += bf16_lo(w[u][i][e]);
              acc[2 * e + 1] += bf16_hi(w[u][i][e]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[u][i][e]);
          }
        }
#pragma unroll
        for (int e = 0; e < kE; ++e) part[(u * kRG + rg) * (D + 1) + ch * kE + e] = acc[e];
      }
      __syncthreads();
      for (int x = tid; x < 2 * D; x += 256) {
        const int u = x / D, d = x % D;
        float sum = 0.f;
#pragma unroll 8
        for (int g = 0; g < kRG; ++g) sum += part[(u * kRG + g) * (D + 1) + d];
        if (r0 + u < kSelRows) qbar[(r0 + u) * D + d] = cnt[u] > 0 ? sum / float(cnt[u]) : 0.f;
      }
      __syncthreads();
    }
  }

  // ---- 2. score
  float a[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) a[j] = ci < R ? qbar[ci * D + kg * kJ + j] : 0.f;
  __syncthreads();  // the score rows overwrite qbar
  {
    auto store = [&](int t, const f32x4& acc) {
      const int n = t * 16 + ci;
      if (t < ntiles && n < ncols) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 4 * kg + v;
          if (r < R) sarea[r * p.rowlen + n + (n >> 5)] = acc[v] * p.scale;
        }
      }
    };
    auto mma_store = [&](int t, const float (&x0)[kJ], const float (&x1)[kJ]) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], x0[j], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], x1[j], acc1, 0, 0, 0);
      }
      store(t, acc0);
      store(t + 4, acc1);
    };
    // two tiles per step (t and t + 4: independent accumulators); the keys of
    // the next step load into the other register set while this one's MFMAs run
    float c0[kJ], c1[kJ];
    for (int t = wave; t < ntiles; t += 16) {
      load_b(t + 8, c0);
      load_b(t + 12, c1);
      mma_store(t, b0, b1);
      if (t + 8 >= ntiles) break;
      load_b(t + 16, b0);
      load_b(t + 20, b1);
      mma_store(t + 8, c0, c1);
    }
  }
  __syncthreads();

  // ---- 3. top-k, one row per wave at a time
  uint32_t* hw = &hist[wave][0][0];
  for (int r = wave; r < R; r += 4) {
    const int m = m0 + r;
    const int n_cand = m + 1;
    const int64_t row = int64_t(bh) * p.NB + m;
    const int k = budget_blocks(n_cand, p.heads.min_blocks[h], p.heads.ratio_q16[h]);
    const int ns = min<int>(p.heads.n_sink[h], n_cand);
    const int nl_lo = max(ns, n_cand - p.heads.n_local[h]);  // forced: [0, ns) U [nl_lo, n_cand)
    const int kk = k - ns - (n_cand - nl_lo);                 // to pick among the others
    int32_t* out = p.idx + row * p.kmax;
    if (lane == 0) p.cnt[row] = k;
    for (int i = k + lane; i < p.kmax; i += 64) out[i] = -1;
    if (kk <= 0 || k == n_cand) {
      // (k >= the forced count: the budget validation keeps min_blocks >=
      // n_sink + n_local; the bounds below only guard the row)
      for (int n = lane; n < n_cand; n += 64) {
        const int at = k == n_cand ? n : n < ns ? n : n >= nl_lo ? ns + (n - nl_lo) : -1;
        if (at >= 0 && at < k) out[at] = n;
      }
      continue;
    }
    const float* srow = sarea + r * p.rowlen;
    const int cr = (n_cand + 63) >> 6;  // candidates per lane this row needs
    if (cr <= 4) topk_row_wave<4, true>(srow, n_cand, k, kk, ns, nl_lo, out, lane, hw);
    else if (cr <= 8) topk_row_wave<8, true>(srow, n_cand, k, kk, ns, nl_lo, out, lane, hw);
    else if (cr <= 16) topk_row_wave<16, true>(srow, n_cand, k, kk, ns, nl_lo, out, lane, hw);
    else topk_row_wave<1, false>(srow, n_cand, k, kk, ns, nl_lo, out, lane, hw);
  }
}

// ---------------------------------------------------------------- top-k
// Exclusive prefix sum (in thread order) of a per-thread count; returns the total.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t& before, uint32_t* red) {
  const int lane = threadIdx.x & 63;
  const uint32_t inc = wave_scan_incl(x);
  const uint32_t wave_tot = uint32_t(__builtin_amdgcn_readlane(int(inc), 63));
  if constexpr (NT == 64) {
    before = inc - x;
    return wave_tot;
  } else {
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 63) red[w] = wave_tot;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      off += (i < w) ? red[i] : 0u;
      tot += red[i];
    }
    before = off + inc - x;
    return tot;
  }
}

// Thread t owns candidates [t*CPT, t*CPT + CPT) of its row.  The kk-th largest
// key among the non-forced candidates is found by a radix select over the four
// bytes of the key (most significant first): a 256-bin histogram of the keys
// that match the bytes fixed so far, then the bin in which the count from the
// top reaches kk.  Keys above the threshold are kept, and of the keys equal to
// it the lowest-index ones; two block-wide scans place the kept candidates in
// index order.
template <int NT, int CPT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkParams p) {
  __shared__ uint32_t red[NT / 64];
  __shared__ uint32_t hist[2][256];
  __shared__ uint32_t found[3];
  __shared__ uint32_t kbuf[NT * CPT + NT * CPT / 32];
  const int row = blockIdx.x;
  if (row >= p.rows) return;
  const int tid = threadIdx.x;
  const int h = row % p.Hq;
  const int n_cand = (p.kv_len + p.heads.gran[h] - 1) / p.heads.gran[h];
  const int k = budget_blocks(n_cand, p.heads.min_blocks[h], p.heads.ratio_q16[h]);
  const int ns = min<int>(p.heads.n_sink[h], n_cand);
  // forced: [0, ns) U [nl_lo, n_cand), the two ranges made disjoint
  const int nl_lo = max(ns, n_cand - p.heads.n_local[h]);
  const int n_forced = ns + (n_cand - nl_lo);
  const int kk = k - n_forced;  // to pick among the others
  int32_t* out = p.idx + (int64_t)row * p.kmax;
  if (tid == 0) p.cnt[row] = k;
  for (int i = k + tid; i < p.kmax; i += NT) out[i] = -1;

  auto forced = [&](int n) { return n < ns || n >= nl_lo; };

  if (kk <= 0 || k == n_cand) {
    // nothing to rank: the forced set (k == |F|) or every candidate (k == n)
    if (k == n_cand) {
      for (int n = tid; n < n_cand; n += NT) out[n] = n;
    } else {
      for (int n = tid; n < n_cand; n += NT) {
        if (n < ns) out[n] = n;
        else if (n >= nl_lo) out[ns + (n - nl_lo)] = n;
      }
    }
    return;
  }

  // keys of the rankable candidates; 0 marks "not rankable" (no float maps to
  // 0).  Read coalesced into LDS (one pad word per 32 keys keeps the per-thread
  // runs on distinct banks), then each thread takes its CPT consecutive keys.
  const float* srow = p.s + (int64_t)row * p.s_row;
  {
    // all CPT loads of a thread issued before any is used (one round trip)
    float v[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) v[c] = srow[min(c * NT + tid, n_cand - 1)];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int n = c * NT + tid;
      kbuf[n + (n >> 5)] = (n < n_cand && !forced(n)) ? ordered_key(v[c]) : 0u;
    }
  }
  __syncthreads();
  const int n0 = tid * CPT;
  uint32_t key[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) key[c] = kbuf[(n0 + c) + ((n0 + c) >> 5)];

  // Radix select on keys relative to the row minimum: rel = key - kmin + 1
  // (0 stays "not rankable").  Digits start at the top set bit of the range,
  // so the first histogram already spreads keys of similar magnitude.
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
    if (key[c] != 0u) {
      kmin = min(kmin, key[c]);
      kmax = max(kmax, key[c]);
    }
  kmin = wave_umin(kmin);
  kmax = wave_umax(kmax);
  if constexpr (NT > 64) {
    __shared__ uint32_t mm[2][NT / 64];
    if ((tid & 63) == 0) {
      mm[0][tid >> 6] = kmin;
      mm[1][tid >> 6] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      kmin = min(kmin, mm[0][i]);
      kmax = max(kmax, mm[1][i]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) key[c] = key[c] != 0u ? key[c] - kmin + 1u : 0u;  // now rel
  const uint32_t range = kmax - kmin + 1u;  // >= 1: kk >= 1 rankable keys exist
  const int bits = 32 - __clz(range);

  uint32_t prefix = 0, pmask = 0, need = (uint32_t)kk;
  uint32_t T = 0, ties_wanted = 0;  // on rel
  int width = bits < 8 ? bits : 8;
  int shift = bits - width;
  // Two barriers per pass: the histograms alternate between two buffers (the
  // one for the next pass is cleared during this one), and wave 0 alone scans
  // the 256 bins (4 per lane, descending digit order) to find the digit.
  for (int i = tid; i < 256; i += NT) hist[0][i] = 0u;
  __syncthreads();
#pragma unroll 1
  for (int pass = 0;; ++pass) {
    uint32_t* const h = hist[pass & 1];
    const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (key[c] != 0u && (key[c] & pmask) == prefix) atomicAdd(&h[(key[c] >> shift) & dmask], 1u);
    __syncthreads();
    if (tid < 64) {
      uint32_t hc[4], loc = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        hc[u] = h[255 - (4 * tid + u)];
        loc += hc[u];
      }
      uint32_t above = wave_scan_incl(loc) - loc;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (above < need && above + hc[u] >= need) {
          found[0] = 255u - uint32_t(4 * tid + u);
          found[1] = need - above;
          found[2] = hc[u];
        }
        above += hc[u];
      }
    }
    for (int i = tid; i < 256; i += NT) hist[(pass + 1) & 1][i] = 0u;
    __syncthreads();
    const uint32_t digit = found[0], rem = found[1], bin = found[2];
    prefix |= digit << shift;
    pmask |= dmask << shift;
    need = rem;
    if (rem == bin && prefix != 0u) {
      // every key of this bin is kept: threshold just below the bin
      T = prefix - 1u;
      ties_wanted = 0;
      break;
    }
    if (shift == 0) {
      T = prefix;
      ties_wanted = rem;
      break;
    }
    width = shift < 8 ? shift : 8;
    shift -= width;
  }
  // One scan of the packed counts (ties << 16 | kept-above) places every kept
  // candidate: the ties taken are the lowest-index ones.
  uint32_t n_tie = 0, n_gt = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int n = n0 + c;
    if (n < n_cand) {
      if (forced(n) || key[c] > T) ++n_gt;
      else if (key[c] == T) ++n_tie;
    }
  }
  uint32_t before;
  block_scan<NT>((n_tie << 16) | n_gt, before, red);
  const uint32_t gt_before = before & 0xffffu, ties_before = before >> 16;
  // ties kept at lower indices, and how many of this thread's ties are kept.
  // Written without a guarded subtraction: ROCm 7.2's clang hoisted the
  // subtraction of a "ties_before >= ties_wanted ? 0 : ties_wanted -
  // ties_before" form out of its guard with its no-wrap flag and then folded
  // min(ties_before, ties_wanted) to ties_before, which misplaced a kept block
  // that had more ties than ties_wanted before it (rows with exact ties).
  const uint32_t taken_before = min(ties_before, ties_wanted);
  const uint32_t my_ties = min(n_tie, ties_wanted - taken_before);
  uint32_t pos = gt_before + taken_before;
  uint32_t t_used = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int n = n0 + c;
    if (n < n_cand) {
      bool take = forced(n) || key[c] > T;
      if (!take && key[c] == T && t_used < my_ties) {
        take = true;
        ++t_used;
      }
      if (take) out[pos++] = n;
    }
  }
}

// ---------------------------------------------------------------- decode scores
// One wave scores rows_per_wg pooled blocks of one (batch, KV head,
// granularity) against every scoring query head of that group and granularity
// (at most MAXH).  The fp32 pooled rows stream through a 4-stage LDS ring
// (8 rows per stage, direct-to-LDS loads, three stages in flight); 16 lanes
// share a row (D/16 floats each) and their partial dots meet by xor-shuffle.
constexpr int kSStages = 4;

template <typename T, int D, int MAXH>
__global__ __launch_bounds__(64) void decode_scores_kernel(DecodeScoreParams p) {
  constexpr int kRowB = D * 4;             // bytes per pooled row
  constexpr int kSR = 8;                   // rows per stage
  constexpr int kStageB = kSR * kRowB;
  constexpr int kInsts = kStageB / 1024;   // 1 KB direct loads per stage
  constexpr int kQ = D / 64;               // 16-byte pieces per lane and row
  static_assert(kInsts * 1024 == kStageB, "stage must fill whole 1 KB loads");
  __shared__ __attribute__((aligned(1024))) char st0[kStageB], st1[kStageB], st2[kStageB], st3[kStageB];
  static_assert(kSStages == 4, "stage variables");
  const DecodeScoreJob& job = p.jobs[blockIdx.y];
  const int bi = blockIdx.z;
  const int lane = threadIdx.x;
  const int sub = lane & 15, rq = lane >> 4;
  const int nc = p.pool_nc[job.pool];
  const int r0 = blockIdx.x * p.rows_per_wg;
  if (r0 >= nc) return;
  const int nr = min(p.rows_per_wg, nc - r0);
  const int n_st = (nr + kSR - 1) / kSR;
  const int nh = job.n_heads;
  const float* kp = p.pooled + p.pool_off[job.pool] + (((int64_t)bi * p.Hkv + job.kvh) * nc + r0) * D;
  const i32x4 rsrc = buffer_rsrc_words(kp, nr * kRowB);  // rows past the chunk read zero

  // query slices: lane holds d = 64 q + 4 sub .. +3 for q < kQ
  f32x4 qv[MAXH][kQ];
#pragma unroll
  for (int i = 0; i < MAXH; ++i) {
    const int hh = job.heads[i < nh ? i : 0];
    const T* qrow = reinterpret_cast<const T*>(p.q) + bi * p.qs0 + hh * p.qs1;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 64 * q + 4 * sub + e;
        if constexpr (sizeof(T) == 2) qv[i][q][e] = bf16_to_f32(qrow[d]);
        else qv[i][q][e] = qrow[d];
      }
  }
  auto stage = [&](auto S) -> char* {
    constexpr int s = decltype(S)::value;
    return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3;
  };
  auto issue = [&](auto S, int si) {
#pragma unroll
    for (int u = 0; u < kInsts; ++u) dma16_stream(rsrc, stage(S) + u * 1024, si * kStageB + u * 1024 + lane * 16);
  };
  float* srow[MAXH];
#pragma unroll
  for (int i = 0; i < MAXH; ++i) srow[i] = p.s + ((int64_t)bi * p.Hq + job.heads[i < nh ? i : 0]) * p.nc_max + r0;

  auto step = [&](auto S, int si) {
    using SN = std::integral_constant<int, (decltype(S)::value + kSStages - 1) % kSStages>;
    if (si + kSStages - 1 < n_st) issue(SN{}, si + kSStages - 1);
    const int after = min(n_st - 1 - si, kSStages - 1);
    if (after >= 3) wait_vmcnt<3 * kInsts>();
    else if (after == 2) wait_vmcnt<2 * kInsts>();
    else if (after == 1) wait_vmcnt<kInsts>();
    else wait_vmcnt<0>();
    const char* sp = stage(S);
#pragma unroll
    for (int pp = 0; pp < kSR / 4; ++pp) {
      const int row = 4 * pp + rq;
      f32x4 kv[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) kv[q] = __builtin_bit_cast(f32x4, lds16(sp, row * kRowB + q * 256 + sub * 16));
      const int r = si * kSR + row;
#pragma unroll
      for (int i = 0; i < MAXH; ++i) {
        if (i >= nh) break;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < kQ; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = fmaf(qv[i][q][e], kv[q][e], acc);
        acc = row_sum16(acc);
        if (sub == 0 && r < nr) srow[i][r] = acc * p.scale;
      }
    }
  };
  issue(std::integral_constant<int, 0>{}, 0);
  if (n_st > 1) issue(std::integral_constant<int, 1>{}, 1);
  if (n_st > 2) issue(std::integral_constant<int, 2>{}, 2);
  for (int i = 0; i < n_st; i += kSStages) {
    step(std::integral_constant<int, 0>{}, i);
    if (i + 1 >= n_st) break;
    step(std::integral_constant<int, 1>{}, i + 1);
    if (i + 2 >= n_st) break;
    step(std::integral_constant<int, 2>{}, i + 2);
    if (i + 3 >= n_st) break;
    step(std::integral_constant<int, 3>{}, i + 3);
  }
}

template <int NT, int CPT>
hipError_t topk_launch(const TopkParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<NT, CPT>), dim3(p.rows), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PoolParams& p, int dtype, int D, int batch, hipStream_t stream) {
  if (p.pages.table && (p.pages.page_size < p.g || p.pages.page_size % p.g || p.pages.max_pages < 1 ||
                        p.pages.pages_per_head < 1))
    return hipErrorInvalidValue;
  dim3 grid((p.nb + p.blocks_per_wg - 1) / p.blocks_per_wg, p.heads, batch);
  const bool nrm = p.norm_max != nullptr;
  if (nrm && p.pages.table) return hipErrorInvalidValue;
  if (dtype == 0 && D == 128) {
    if (nrm) hipLaunchKernelGGL((pool_kernel<bf16_t, 128, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((pool_kernel<bf16_t, 128, false>), grid, dim3(256), 0, stream, p);
  } else if (dtype == 0 && D == 64) {
    if (nrm) hipLaunchKernelGGL((pool_kernel<bf16_t, 64, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((pool_kernel<bf16_t, 64, false>), grid, dim3(256), 0, stream, p);
  } else if (dtype == 1 && D == 128) {
    if (nrm) hipLaunchKernelGGL((pool_kernel<float, 128, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((pool_kernel<float, 128, false>), grid, dim3(256), 0, stream, p);
  } else if (dtype == 1 && D == 64) {
    if (nrm) hipLaunchKernelGGL((pool_kernel<float, 64, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((pool_kernel<float, 64, false>), grid, dim3(256), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t select_prefill_launch(const PrefillSelectParams& p, int block, int batch, hipStream_t stream) {
  const dim3 grid(batch * p.Hq * p.n_mg);
  if (block == 128) hipLaunchKernelGGL((select_prefill_kernel<T, D, 128>), grid, dim3(256), 0, stream, p);
  else if (block == 64) hipLaunchKernelGGL((select_prefill_kernel<T, D, 64>), grid, dim3(256), 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_select_prefill(const PrefillSelectParams& p, int dtype, int D, int block, int batch,
                                 hipStream_t stream) {
  if (p.NB < 1 || p.NB > kSelMaxBlocks || p.R != sel_rows(p.NB) || p.rowlen != sel_rowlen(p.NB) ||
      p.n_mg != (p.NB + p.R - 1) / p.R)
    return hipErrorInvalidValue;
  if (dtype == 0 && D == 128) return select_prefill_launch<bf16_t, 128>(p, block, batch, stream);
  if (dtype == 0 && D == 64) return select_prefill_launch<bf16_t, 64>(p, block, batch, stream);
  if (dtype == 1 && D == 128) return select_prefill_launch<float, 128>(p, block, batch, stream);
  if (dtype == 1 && D == 64) return select_prefill_launch<float, 64>(p, block, batch, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const TopkParams& p, int max_cand, hipStream_t stream) {
  // decode rows are few (batch x heads): wide workgroups, few keys per thread
  if (max_cand <= 256) return topk_launch<256, 1>(p, stream);
  if (max_cand <= 1024) return topk_launch<256, 4>(p, stream);
  if (max_cand <= 2048) return topk_launch<256, 8>(p, stream);
  if (max_cand <= 4096) return topk_launch<512, 8>(p, stream);
  if (max_cand <= 8192) return topk_launch<1024, 8>(p, stream);
  if (max_cand <= 16384) return topk_launch<1024, 16>(p, stream);
  return hipErrorInvalidValue;
}

template <int MAXH>
hipError_t decode_scores_launch(const DecodeScoreParams& p, int dtype, int D, dim3 grid, hipStream_t stream) {
  if (dtype == 0 && D == 128) hipLaunchKernelGGL((decode_scores_kernel<bf16_t, 128, MAXH>), grid, dim3(64), 0, stream, p);
  else if (dtype == 0 && D == 64) hipLaunchKernelGGL((decode_scores_kernel<bf16_t, 64, MAXH>), grid, dim3(64), 0, stream, p);
  else if (dtype == 1 && D == 128) hipLaunchKernelGGL((decode_scores_kernel<float, 128, MAXH>), grid, dim3(64), 0, stream, p);
  else if (dtype == 1 && D == 64) hipLaunchKernelGGL((decode_scores_kernel<float, 64, MAXH>), grid, dim3(64), 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_scores(const DecodeScoreParams& p, int dtype, int D, int batch, hipStream_t stream) {
  int max_nc = 0, max_h = 1;
  for (int i = 0; i < 4; ++i) max_nc = max(max_nc, p.pool_nc[i]);
  for (int i = 0; i < p.n_jobs; ++i) max_h = max(max_h, p.jobs[i].n_heads);
  dim3 grid((max_nc + p.rows_per_wg - 1) / p.rows_per_wg, p.n_jobs, batch);
  if (max_h <= 2) return decode_scores_launch<2>(p, dtype, D, grid, stream);
  if (max_h <= 4) return decode_scores_launch<4>(p, dtype, D, grid, stream);
  if (max_h <= 8) return decode_scores_launch<8>(p, dtype, D, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
