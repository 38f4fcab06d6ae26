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
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  constexpr int kE = 16 / int(sizeof(T));  // elements per chunk
  constexpr int kCh = D / kE;              // chunks per row
  constexpr int kRG = 256 / kCh;           // row groups
  __shared__ float part[kRG][D + 1];
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
    for (int r = rg; r < cnt; r += kRG) {
      // read once: non-temporal, so the rows are not kept in the caches
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (int64_t)(lo + r) * rs + ch * 16));
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_lo(w[e]);
          acc[2 * e + 1] += bf16_hi(w[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
      }
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
    __syncthreads();
  }
}

// ---------------------------------------------------------------- prefill block scores
// s[bh][m][n] = scale * <Qbar[bh][m], Kbar[bkv][n]> for the causal 128x128
// tiles, in fp32 on the MFMA pipe (v_mfma_f32_32x32x2f32; each wave one 64x64
// quadrant as 2x2 MFMA tiles).  fp32 keeps the scores exact enough for the
// 1e-4 relative gaps the selection is checked against.  Qbar and Kbar rows are
// staged through LDS in 32-wide d chunks, shared by the four waves.
constexpr int kScoreTile = 128;

template <int D>
__global__ __launch_bounds__(256) void prefill_scores_kernel(PrefillScoreParams p) {
  constexpr int kT = kScoreTile;
  constexpr int kDC = 32;  // d columns staged per pass
  __shared__ float qs[kT][kDC + 1];
  __shared__ float ks[kT][kDC + 1];
  const int n0 = blockIdx.x * kT, m0 = blockIdx.y * kT;
  if (n0 > m0 + kT - 1) return;  // entirely above the diagonal
  const int bh = blockIdx.z;
  const int bi = bh / p.Hq, h = bh % p.Hq;
  const int bkv = bi * (p.Hq / p.G) + h / p.G;
  const float* qp = p.qp + (int64_t)bh * p.NB * D;
  const float* kp = p.kp + (int64_t)bkv * p.NB * D;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int mi = wave >> 1, ni = wave & 1;  // this wave's 64 x 64 quadrant
  const int col = lane & 31, kh = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
  for (int d0 = 0; d0 < D; d0 += kDC) {
    f32x4 va[kT * kDC / 4 / 256], vb[kT * kDC / 4 / 256];
#pragma unroll
    for (int u = 0; u < kT * kDC / 4 / 256; ++u) {
      const int i = u * 256 + tid;
      const int r = i / (kDC / 4), c = (i % (kDC / 4)) * 4;
      va[u] = (m0 + r < p.NB) ? *reinterpret_cast<const f32x4*>(qp + (int64_t)(m0 + r) * D + d0 + c) : f32x4{};
      vb[u] = (n0 + r < p.NB) ? *reinterpret_cast<const f32x4*>(kp + (int64_t)(n0 + r) * D + d0 + c) : f32x4{};
    }
#pragma unroll
    for (int u = 0; u < kT * kDC / 4 / 256; ++u) {
      const int i = u * 256 + tid;
      const int r = i / (kDC / 4), c = (i % (kDC / 4)) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qs[r][c + e] = va[u][e];
        ks[r][c + e] = vb[u][e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kDC; kk += 2) {
      float av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = qs[mi * 64 + t * 32 + col][kk + kh];
        bv[t] = ks[ni * 64 + t * 32 + col][kk + kh];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
  // acc[a][b][i] holds row 8 (i / 4) + 4 kh + i % 4 of row tile a, column col of column tile b
  float* sbase = p.s + (int64_t)bh * p.NB * p.NB;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int n = n0 + ni * 64 + b * 32 + col;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + mi * 64 + a * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
        if (m < p.NB && n <= m) sbase[(int64_t)m * p.NB + n] = acc[a][b][i] * p.scale;
      }
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
  int h, n_cand;
  if (p.mode == 0) {
    const int m = row % p.NB;
    h = (row / p.NB) % p.Hq;
    n_cand = m + 1;
  } else {
    h = row % p.Hq;
    const int g = p.heads.gran[h];
    n_cand = (p.kv_len + g - 1) / g;
  }
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
  if (dtype == 0 && D == 128) hipLaunchKernelGGL((pool_kernel<bf16_t, 128>), grid, dim3(256), 0, stream, p);
  else if (dtype == 0 && D == 64) hipLaunchKernelGGL((pool_kernel<bf16_t, 64>), grid, dim3(256), 0, stream, p);
  else if (dtype == 1 && D == 128) hipLaunchKernelGGL((pool_kernel<float, 128>), grid, dim3(256), 0, stream, p);
  else if (dtype == 1 && D == 64) hipLaunchKernelGGL((pool_kernel<float, 64>), grid, dim3(256), 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill_scores(const PrefillScoreParams& p, int D, int batch, hipStream_t stream) {
  const int t = (p.NB + kScoreTile - 1) / kScoreTile;
  dim3 grid(t, t, batch * p.Hq);
  if (D == 128) hipLaunchKernelGGL((prefill_scores_kernel<128>), grid, dim3(256), 0, stream, p);
  else if (D == 64) hipLaunchKernelGGL((prefill_scores_kernel<64>), grid, dim3(256), 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, int max_cand, hipStream_t stream) {
  if (p.mode == 0) {
    if (max_cand <= 64) return topk_launch<64, 1>(p, stream);
    if (max_cand <= 128) return topk_launch<64, 2>(p, stream);
    if (max_cand <= 256) return topk_launch<64, 4>(p, stream);
    if (max_cand <= 512) return topk_launch<64, 8>(p, stream);
    if (max_cand <= 1024) return topk_launch<64, 16>(p, stream);
    if (max_cand <= 2048) return topk_launch<64, 32>(p, stream);
    if (max_cand <= 4096) return topk_launch<256, 16>(p, stream);
    if (max_cand <= 8192) return topk_launch<256, 32>(p, stream);
  } else {
    // decode rows are few (batch x heads): wide workgroups, few keys per thread
    if (max_cand <= 256) return topk_launch<256, 1>(p, stream);
    if (max_cand <= 1024) return topk_launch<256, 4>(p, stream);
    if (max_cand <= 2048) return topk_launch<256, 8>(p, stream);
    if (max_cand <= 4096) return topk_launch<512, 8>(p, stream);
    if (max_cand <= 8192) return topk_launch<1024, 8>(p, stream);
    if (max_cand <= 16384) return topk_launch<1024, 16>(p, stream);
  }
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
