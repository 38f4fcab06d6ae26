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
//   workgroup = B/32 waves; wave w owns query rows [32w, 32w+32) of the tile.
//   step      = 64 keys of one selected key block (B/64 steps per block).
//   Every step's K and V rows are gathered through the block-index table with
//   buffer loads straight into LDS (buffer_load_dwordx4 ... lds: no registers;
//   the (batch, KV head) slice is the buffer, so rows past the sequence end
//   read as zero).  K and V live in two-slot LDS rings; K runs one step ahead
//   of V.  Iteration i, after one barrier, fetches K(i+2) and V(i+1), computes
//   S(i+1) = K(i+1) Q^T on the MFMA pipe while the VALU turns S(i) into P(i),
//   then accumulates O += P(i) V(i).
//
// Math per step and wave (bf16):
//   S^T[key][q] = K Q^T    v_mfma_f32_32x32x16_bf16, A = K rows (LDS), B = Q^T
//                          (registers, one load per tile).  Each lane column is
//                          one query, so the row max and row sum are in-lane
//                          plus one exchange between the two half-waves.
//   O^T[d][q] += V^T P^T   A = V^T fragments read with ds_read_b64_tr_b16
//                          (V stays row-major in LDS), B = P^T straight from
//                          the S^T accumulators: key rows are stored in LDS with
//                          bits 2 and 3 of the key index swapped, so lane
//                          element i of S^T holds key 16*(i/8) + 8*half + i%8,
//                          8 consecutive keys per 16-key chunk as the B operand
//                          wants.
//   fp32 inputs: v_mfma_f32_32x32x2f32 with the same layouts, P kept in fp32,
//   V^T elements read one by one.
// Softmax: scores stay unscaled; p = exp2(s*c - m) with c = scale*log2(e) is one
// FMA and one v_exp_f32.  The running max m is raised only when a score exceeds it by more
// than 2^kLazy (decided per wave; O and l are then rescaled), so p <= 2^kLazy;
// l and O share m, so the quotient is unchanged.

#include <climits>

#include "sa_device.hpp"
#include "sa_kernels.hpp"
#include "sa_prefill_common.hpp"

namespace sa {

namespace {

using namespace prefill;

// A step of the cursor with the global byte addresses of its (batch, KV head)
// K and V slices, computed once when the cursor enters a tile so that a
// step's gathers only add the row offset.
struct StepAt : Step {
  uint64_t ka, va;
};

// log2 headroom a score may have over the running max before P could grow
// past 2^kSafe; with P <= 2^64 neither P, the row sum nor O can overflow fp32
// for any |v| below 1e13 over up to 2^20 keys.
constexpr float kSafe = 64.f;

template <typename T, int D, int B, bool kLse>
__global__ __launch_bounds__(2 * B) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillParams p) {
  using C = Cfg<T, D, B>;
  __shared__ __attribute__((aligned(1024))) char smem[C::kLds];
  char* const kring = smem;                 // K slots 0, 1
  char* const vring = smem + 2 * C::kTile;  // V slots 0, 1

  wg_stamp(0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;   // MFMA column (query) / A-row (key, d) index
  const int half = lane >> 5;  // MFMA k-half

  // Work queue (p.queue set): the workgroups take the items of a global list
  // in order, each claiming its next item from a counter when it starts the
  // current one, so faster compute units simply take more items.  The list may
  // be cut into partitions, one counter each (one per XCD, so that the
  // workgroups of an XCD share its L2): a workgroup starts on partition
  // blockIdx.x % n_queues and, once that is empty, moves on to the following
  // ones in turn; after trying every partition it is done.  Wave 0 makes the
  // claims and hands each to the other waves through LDS; its partition and
  // the partitions left to try sit in LDS (q_state), out of the registers of
  // the main loop.
  __shared__ int q_slot;
  __shared__ int q_state[2];  // wave 0: current partition, partitions left
  int q_pend = 0;             // wave 0, lane 0: the claim in flight
  auto claim = [&]() {
    if (wave == 0 && lane == 0 && q_state[1] > 0) q_pend = atomicAdd(COLD(queue) + q_state[0], 1);
  };
  // position in items_by_bin of the claim in flight (n_tiles: none left)
  auto take_claim = [&]() -> int {
    __syncthreads();  // every wave has read the previous claim
    if (wave == 0) {
      const int n_tiles = COLD(n_tiles), nq = COLD(n_queues);
      int qc = __builtin_amdgcn_readfirstlane(q_state[0]);
      int left = __builtin_amdgcn_readfirstlane(q_state[1]);
      int v = __builtin_amdgcn_readfirstlane(q_pend);
      int pos = n_tiles;
      while (left > 0) {  // at most n_queues rounds per workgroup in all
        const int beg = min(max(kernel_arg<int>(offsetof(PrefillParams, qoff) + 4 * qc), 0), n_tiles);
        const int end = min(max(kernel_arg<int>(offsetof(PrefillParams, qoff) + 4 * qc + 4), beg), n_tiles);
        if (v < end - beg) {
          pos = beg + v;
          break;
        }
        if (--left == 0) break;
        qc = qc + 1 == nq ? 0 : qc + 1;
        if (lane == 0) q_pend = atomicAdd(COLD(queue) + qc, 1);
        v = __builtin_amdgcn_readfirstlane(q_pend);
      }
      if (lane == 0) {
        q_slot = pos;
        q_state[0] = qc;
        q_state[1] = left;
      }
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(q_slot);
  };
  const bool qmode = p.queue != nullptr;

  int it_beg, it_end;
  if (qmode) {
    if (wave == 0 && lane == 0) {
      q_state[0] = blockIdx.x % p.n_queues;
      q_state[1] = p.n_queues;
    }
    claim();
    it_beg = take_claim();
    claim();
    it_end = p.n_tiles;  // positions in the global list
  } else if (p.bin_offsets) {
    it_beg = p.bin_offsets[blockIdx.x];
    it_end = p.bin_offsets[blockIdx.x + 1];
  } else {
    it_beg = blockIdx.x;
    it_end = (int)blockIdx.x < p.n_tiles ? (int)blockIdx.x + 1 : (int)blockIdx.x;
  }
  const int S = p.S;
  const float c2 = p.scale_log2;
  const int krs = int(p.ks2 * (int64_t)sizeof(T));
  const int vrs = int(p.vs2 * (int64_t)sizeof(T));

  // ---------------------------------------------------------------- step cursor
  // The bin's items and each tile's block list are read through per-wave
  // register windows (lane l holds entry base + l) and picked out with
  // readlane, so advancing a step never waits on memory.  The window of the
  // next item's blocks is fetched while the current item runs.
  int ibase = it_beg;
  int iw_tile = -1, iw_cnt = 0;  // per lane: tile and block count of item ibase + lane
  auto load_items = [&](int base) {
    ibase = base;
    const int it = base + lane;
    int t = -1, c = 0;
    if (it < it_end) {
      const int32_t* items = COLD(items_by_bin);
      t = items ? items[it] : it;
      if (t >= 0 && t < COLD(n_tiles)) c = min(COLD(block_cnt)[t], COLD(kmax));
      else t = -1;
    }
    iw_tile = t;
    iw_cnt = c;
  };
  auto load_blocks = [&](int tile, int cnt, int base) {
    const int jj = base + lane;
    return jj < cnt ? COLD(block_idx)[(int64_t)tile * COLD(kmax) + jj] : -1;
  };
  // queue mode: tile and block count of the item at position it
  auto queue_item = [&](int it, int& tile, int& cnt) {
    tile = COLD(items_by_bin)[it];
    if (tile >= 0 && tile < COLD(n_tiles)) {
      cnt = min(COLD(block_cnt)[tile], COLD(kmax));
    } else {
      tile = -1;
      cnt = 0;
    }
  };
  // cursor over the lookahead step (the others are copies of it)
  int c_cnt = 0, c_wbase = 0, c_win = -1;  // blocks of the cursor's tile: window at c_wbase
  int nx_item = -1, nx_win = -1;            // prefetched first window of item nx_item
  int nx_tile = -1, nx_cnt = 0;             // queue mode: its tile and block count
  int q_next = 0;                           // queue mode: the item after the cursor's
  StepAt cur;
  cur.valid = 0;
  const float* const knorm = p.key_norms;  // nullable

  auto item_tile = [&](int it, int& tile, int& cnt) {
    if (qmode) {
      if (it == nx_item) {
        tile = nx_tile;
        cnt = nx_cnt;
      } else {
        queue_item(it, tile, cnt);
      }
      return;
    }
    if (it - ibase >= 64) load_items(it);
    tile = __builtin_amdgcn_readlane(iw_tile, it - ibase);
    cnt = __builtin_amdgcn_readlane(iw_cnt, it - ibase);
  };
  auto prefetch_next = [&](int it) {
    nx_item = -1;
    if (it >= it_end) return;
    int tile, cnt;
    if (qmode) {
      queue_item(it, tile, cnt);
    } else {
      if (it - ibase >= 64) return;
      tile = __builtin_amdgcn_readlane(iw_tile, it - ibase);
      cnt = __builtin_amdgcn_readlane(iw_cnt, it - ibase);
    }
    if (tile < 0) return;
    nx_win = load_blocks(tile, cnt, 0);
    nx_item = it;
    nx_tile = tile;
    nx_cnt = cnt;
  };
  // first valid block at or after position j of item `it` (moving to later items)
  auto seek = [&](int it, int j) {
    while (true) {
      if (it >= it_end) {
        cur.valid = 0;
        return;
      }
      if (it != cur.item || !cur.valid) {
        int tile, cnt;
        item_tile(it, tile, cnt);
        cur.item = it;
        cur.valid = 1;
        cur.tile = tile;
        c_cnt = tile >= 0 ? cnt : 0;
        c_wbase = 0;
        if (qmode) {
          q_next = take_claim();  // claimed when the previous item started
          claim();
        }
        if (tile >= 0) {
          c_win = (nx_item == it) ? nx_win : load_blocks(tile, c_cnt, 0);
          const int NB = COLD(NB), Hq = COLD(Hq);
          cur.m = tile % NB;
          cur.bh = tile / NB;
          const int kb = cur.bh / Hq, kh = (cur.bh % Hq) / COLD(G);
          cur.ka = reinterpret_cast<uint64_t>(COLD(k)) + (kb * COLD(ks0) + kh * COLD(ks1)) * (int64_t)sizeof(T);
          cur.va = reinterpret_cast<uint64_t>(COLD(v)) + (kb * COLD(vs0) + kh * COLD(vs1)) * (int64_t)sizeof(T);
          prefetch_next(qmode ? q_next : it + 1);
        }
      }
      for (; j < c_cnt; ++j) {
        if (j - c_wbase >= 64) {
          c_wbase = j;
          c_win = load_blocks(cur.tile, c_cnt, j);
        }
        const int n = __builtin_amdgcn_readlane(c_win, j - c_wbase);
        if (n >= 0 && n <= cur.m) {
          cur.j = j;
          cur.hs = 0;
          cur.n = n;
          return;
        }
      }
      it = qmode ? q_next : it + 1;
      j = 0;
    }
  };
  auto advance = [&]() {
    if (!cur.valid) return;
    if (cur.hs + 1 < C::kNSub) {
      cur.hs += 1;
      return;
    }
    seek(cur.item, cur.j + 1);
  };

  // ---------------------------------------------------------------- direct loads
  // Wave instruction t of a step fills LDS bytes [1024 t, 1024 t + 1024): lane i
  // writes 16 bytes at 1024 t + 16 i, i.e. LDS row r = (1024 t + 16 i) / kRow,
  // physical chunk cp; it fetches the global row and chunk the swizzle puts there.
  int k_voff[C::kInstsPerWave], v_voff[C::kInstsPerWave];
#pragma unroll
  for (int u = 0; u < C::kInstsPerWave; ++u) {
    const int t = wave * C::kInstsPerWave + u;
    const int byte = t * 1024 + lane * 16;
    const int r = byte / C::kRow, cp = (byte % C::kRow) / 16;
    k_voff[u] = perm_key(r) * krs + (cp ^ C::swz_k(r)) * 16;
    v_voff[u] = r * vrs + (cp ^ C::swz_v(r)) * 16;
  }
  // The buffer starts at the step's first key row and ends at the sequence
  // end, so the per-lane offsets stay fixed (no per-step vector arithmetic)
  // and rows past the end read as zero.  The loads are issued from inline
  // assembly: the compiler then does not make the fragment reads of the other
  // ring slots wait for them, so each step's gathers have a whole step to
  // land; the wait and barrier at the top of the next iteration order them
  // before their slots are read.
  // this wave's share of each LDS slot starts kInstsPerWave KB into it
  const uint32_t lds_wave =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)smem)) + wave * C::kInstsPerWave * 1024;
  auto fetch = [&](const StepAt& s, int slot, bool k_side) {
    const int rs = k_side ? krs : vrs;
    const int row = s.n * B + s.hs * kKS;
    const i32x4 r = buffer_rsrc_words(reinterpret_cast<const char*>(k_side ? s.ka : s.va) + (int64_t)row * rs,
                                      max(S - row, 0) * rs);
    const uint32_t lw = __builtin_amdgcn_readfirstlane(lds_wave);
    // smem: K slots 0, 1, then V slots 0, 1
    const int* vo = k_side ? k_voff : v_voff;
    const int which = (k_side ? 0 : 2) + slot;
    if (which == 0) dma16_async_run<0, C::kInstsPerWave>(r, lw, vo);
    else if (which == 1) dma16_async_run<C::kTile, C::kInstsPerWave>(r, lw, vo);
    else if (which == 2) dma16_async_run<2 * C::kTile, C::kInstsPerWave>(r, lw, vo);
    else dma16_async_run<3 * C::kTile, C::kInstsPerWave>(r, lw, vo);
  };
  // all of this wave's direct loads have landed in LDS (vmcnt(0) only)
  auto wait_loads = [&]() { wait_vmcnt<0>(); };

  // ---------------------------------------------------------------- tile state
  u32x4 qf[C::kDG];  // Q^T fragments of the wave's 32 queries
  f32x16 oacc[C::kDT];
  // l_run: sum of the probabilities exactly as the P V MFMAs weight the V rows
  // (bf16-rounded for bf16 inputs), so O / l_run is a convex combination of V
  // rows with those weights; l_lse: the same sum before rounding, for lse only.
  float m_run = kNegInf, l_run = 0.f, l_lse = 0.f;
  // With a key-norm table: |score| <= |q| * (the block's key-norm bound), so
  // a step whose bound times qn_c2 = scale * log2(e) * |q| stays within kSafe
  // of the running max for every row needs no row max (P <= 2^kSafe).
  // kn_lim: the largest key-norm bound (bf16 bits, rounded down) for which
  // that holds in every row of the wave, -1 when none (the row max is then
  // taken).
  float qn_c2 = 0.f;
  int kn_lim = -1;
  int t_knb = 0;  // key-norm table row of the tile's (batch, KV head)
  int t_bh = 0, t_m = 0;  // tile being accumulated

  auto start_tile = [&](const StepAt& s) {
    t_bh = s.bh;
    t_m = s.m;
    const int Hq = COLD(Hq);
    const int bi = s.bh / Hq, h = s.bh % Hq;
    const int qrow = s.m * B + wave * 32 + col;
    const char* rp = reinterpret_cast<const char*>(COLD(q)) +
                     (bi * COLD(qs0) + h * COLD(qs1) + (int64_t)qrow * COLD(qs2)) * (int64_t)sizeof(T);
#pragma unroll
    for (int dg = 0; dg < C::kDG; ++dg) {
      // bf16: lane half g holds d = 16*dg + 8*g .. +7; fp32: d = 8*dg + 4*g .. +3
      const int d0 = dg * 2 * C::kE16 + half * C::kE16;
      qf[dg] = qrow < S ? *reinterpret_cast<const u32x4*>(rp + d0 * (int)sizeof(T)) : u32x4{0u, 0u, 0u, 0u};
    }
    m_run = kNegInf;
    l_run = 0.f;
    l_lse = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) oacc[dt] = f32x16{};
    kn_lim = -1;
    if (knorm) {
      const int G = COLD(G);
      t_knb = ((s.bh / Hq) * (Hq / G) + (s.bh % Hq) / G) * COLD(NB);
      float q2 = 0.f;
#pragma unroll
      for (int dg = 0; dg < C::kDG; ++dg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (C::kBf16) {
            // plain FMAs (a v_dot2 chain over vector elements is mis-folded
            // by ROCm 7.2's compiler)
            const float lo = bf16_lo(qf[dg][e]), hi = bf16_hi(qf[dg][e]);
            q2 = fmaf(lo, lo, fmaf(hi, hi, q2));
          } else {
            const float x = __uint_as_float(qf[dg][e]);
            q2 = fmaf(x, x, q2);
          }
        }
      qn_c2 = __builtin_sqrtf(sum_xor32(q2)) * c2;
    }
  };

  auto finish_tile = [&]() {
    const int Hq = COLD(Hq);
    const int bi = t_bh / Hq, h = t_bh % Hq;
    const float l = sum_xor32(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lx = kLse && C::kBf16 ? sum_xor32(l_lse) : l;
    const int qrow = t_m * B + wave * 32 + col;
    if (qrow < S) {
      const int64_t orow = bi * COLD(os0) + h * COLD(os1) + (int64_t)qrow * COLD(os2);
      void* const out = COLD(o);
      const bool out_f32 = COLD(out_f32);
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = dt * 32 + r4 * 8 + half * 4;
          const float o0 = oacc[dt][r4 * 4 + 0] * inv, o1 = oacc[dt][r4 * 4 + 1] * inv;
          const float o2 = oacc[dt][r4 * 4 + 2] * inv, o3 = oacc[dt][r4 * 4 + 3] * inv;
          if (C::kBf16 && !out_f32) {
            *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(out) + orow + d) =
                uint2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + orow + d) = f32x4{o0, o1, o2, o3};
          }
        }
      }
      float* const lse = COLD(lse);
      if (kLse && half == 0) lse[(int64_t)t_bh * S + qrow] = lx > 0.f ? (m_run + __log2f(lx)) * kLn2 : kNegInf;
    }
  };

  // S^T = K Q^T of a step from K slot `slot`
  auto qk = [&](int slot, f32x16(&sacc)[2]) {
    const char* ks = kring + slot * C::kTile;
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int dg = 0; dg < C::kDG; ++dg) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int r = kt * 32 + col;
        const u32x4 a = lds16(ks, r * C::kRow + ((dg * 2 + half) ^ C::swz_k(r)) * 16);
        if constexpr (C::kBf16) {
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, qf[dg]), sacc[kt], 0, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(qf[dg][e]),
                                                            sacc[kt], 0, 0, 0);
        }
      }
    }
  };

  // Masking of a step's scores in place (causal diagonal, sequence tail, or a
  // step this wave cannot see at all).
  auto apply_mask = [&](const StepAt& s, f32x16(&sacc)[2]) {
    const int key0 = s.hs * kKS;
    const bool diag = s.n == s.m;
    const int q_in_blk = wave * 32 + col;
    // straight-line selects (no per-element branches): the first masked key of
    // this lane's query row, then one compare per score
    const int lim = min(diag ? q_in_blk : B, S - s.n * B - 1);  // largest visible key of the block
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kl = key0 + kt * 32 + (i >> 3) * 16 + half * 8 + (i & 7);
        sacc[kt][i] = kl > lim ? kNegInf : sacc[kt][i];
      }
  };

  // One step: S(i+1) = K(i+1) Q^T (K slot slot^1) issued on the MFMA pipe,
  // interleaved with the VALU turning S(i) into P(i), then O += P(i) V(i)
  // (V slot `slot`).  Straight-line; the running max is final for S(i).
  auto fused = [&](int slot, f32x16(&sc)[2], f32x16(&sn)[2]) {
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    const char* ks = kring + (slot ^ 1) * C::kTile;
    const char* vs = vring + slot * C::kTile;
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    if constexpr (C::kBf16) {
      // the wave in its MFMA section issues ahead of a wave that is waiting,
      // fetching or advancing its cursor, so the MFMA pipe stays fed
      __builtin_amdgcn_s_setprio(1);
      u32x4 pf[4];
      float ps0 = 0.f, ps1 = 0.f, px0 = 0.f, px1 = 0.f;
      const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int dg = 0; dg < C::kDG; ++dg) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int r = kt * 32 + col;
          const u32x4 a = lds16(ks, r * C::kRow + ((dg * 2 + half) ^ C::swz_k(r)) * 16);
          sn[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, qf[dg]), sn[kt], 0, 0, 0);
        }
        // a share of this lane's 32 probabilities per k-group
#pragma unroll
        for (int w2 = 0; w2 < 16 / C::kDG; ++w2) {
          const int pair = dg * (16 / C::kDG) + w2;  // 0..15
          const int kc = pair >> 2, w = pair & 3;
          const int i = (kc & 1) * 8 + 2 * w;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kc >> 1][i], c2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kc >> 1][i + 1], c2, -m_use));
          const uint32_t pk = pack_bf16x2(p0, p1);
          pf[kc][w] = pk;
          // the rounded pair summed in one v_dot2 against (1, 1): products
          // exact, fp32 sum; two chains.  Taken on the packed word itself (a
          // dot product on the fragment vector after it is built was folded
          // wrongly by the compiler, reading some words twice)
          if (w2 & 1) ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one2, ps1, false);
          else ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one2, ps0, false);
          if constexpr (kLse) {
            px0 += p0;
            px1 += p1;
          }
        }
      }
      l_run += ps0 + ps1;
      if constexpr (kLse) l_lse += px0 + px1;
      // O^T += V^T P^T.  A fragments by transposed LDS reads: 16-lane group G
      // covers d = 32 dt + 16 (G % 2) + lane % 16 and keys 16 kc + 8 (G / 2) +
      // 4 r + 0..3; source lane j of the group points at V row k0 + j / 4,
      // columns dbase + 4 (j % 4) .. +3.
      const int G = lane >> 4, j = lane & 15;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) {
          const int d = dt * 32 + (G & 1) * 16 + (j & 3) * 4;
          const int row0 = kc * 16 + (G >> 1) * 8 + (j >> 2);
          const int row1 = row0 + 4;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(vs + row0 * C::kRow + (((d >> 3) ^ C::swz_v(row0)) << 4) + ((d & 7) << 1)));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(vs + row1 * C::kRow + (((d >> 3) ^ C::swz_v(row1)) << 4) + ((d & 7) << 1)));
          const u32x4 a = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, pf[kc]), oacc[dt], 0, 0, 0);
        }
      }
      // Issue order: K fragment reads run four MFMAs ahead; the Q K^T MFMAs
      // go out nearly back to back (one VALU op behind each at D = 128), and
      // every P V MFMA carries the transposed V reads of the MFMA two places
      // later and most of the softmax VALU (eight ops at D = 128), so the
      // MFMA pipe runs under the VALU work and LDS latency stays hidden.
      // Measured on the 128K layer, one process: 1 / 8 VALU ops per Q K^T /
      // P V MFMA 9.04 ms, 1 / 9, 1 / 10 and 0 / 8 within 0.3% of it, 1 / 7
      // 9.33, 2 / 9 9.56, against 10.30 for the former 6 / 3 with the row
      // sum taken by unpacking and adding the rounded pair.
      constexpr int kQkValu = 128 / D, kPvValu = 8 * 128 / D;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int u = 0; u < 2 * C::kDG; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, kQkValu, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int u = 0; u < 4 * C::kDT; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read (transposed)
        __builtin_amdgcn_sched_group_barrier(0x003, kPvValu, 0);  // VALU
      }
      __builtin_amdgcn_s_setprio(0);
    } else {
      qk(slot ^ 1, sn);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sc[kt][i], c2, -m_use));
          sc[kt][i] = pv;
          psum += pv;
        }
      l_run += psum;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) {
          const int d = dt * 32 + col;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int row = kc * 16 + half * 8 + e;
            const int off = row * C::kRow + (((d >> 2) ^ C::swz_v(row)) << 4) + ((d & 3) << 2);
            const float a = *reinterpret_cast<const float*>(vs + off);
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sc[kc >> 1][(kc & 1) * 8 + e], oacc[dt], 0, 0, 0);
          }
        }
      }
    }
  };

  // ---------------------------------------------------------------- walk
  // Step i's K sits in K slot i%2, its V in V slot i%2.  At the top of
  // iteration i, S(i) is computed and K(i+1), V(i) were fetched during
  // iteration i-1.
  load_items(it_beg);
  cur.item = -1;
  seek(it_beg, 0);
  StepAt s0 = cur;
  if (!s0.valid) {
    wg_stamp(1);
    return;
  }
  advance();
  StepAt s1 = cur;
  advance();
  fetch(s0, 0, true);
  fetch(s0, 0, false);
  if (s1.valid) fetch(s1, 1, true);
  wait_loads();
  __syncthreads();
  start_tile(s0);
  f32x16 sa[2], sb[2];
  qk(0, sa);

  auto iteration = [&](int slot, f32x16(&sc)[2], f32x16(&sn)[2]) -> bool {
    // the step's key-norm bound (bf16 bits rounded up; 0x7fff: no table),
    // issued before the barrier so that its latency hides behind it (a scalar
    // load, through the constant address space: a vector load would be waited
    // for with vmcnt(0), which also waits for the gathers)
    const uint32_t kn_raw = knorm ? ((const __attribute__((address_space(4))) uint32_t*)(uintptr_t)knorm)[t_knb + s0.n]
                                  : 0x7fff0000u;
    // K(i+1) and V(i) are in LDS; every wave is done with the slots refilled here
    wait_loads();
    __syncthreads();
    if (cur.valid) fetch(cur, slot, true);  // K(i+2)
    if (s1.valid) fetch(s1, slot ^ 1, false);  // V(i+1)
    const bool pipe = s1.valid && s1.item == s0.item;
    // rare: masking (causal diagonal, tail, or an invisible step)
    const int key0 = s0.hs * kKS;
    const bool masked = (s0.n == s0.m && key0 + kKS - 1 > wave * 32) || s0.n * B + key0 + kKS > S;
    if (masked) apply_mask(s0, sc);
    // rare: the row max and raising the running max (always at the first
    // step of a tile; with a key-norm table only where the bound allows more
    // than kSafe over the running max)
    const int kn0 = int((kn_raw + 0xffffu) >> 16);
    if (kn0 > kn_lim) {
      // row max: one v_max3 per pair of scores
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, sc[kt][i]), sc[kt][i + 1]);
      mx = max_xor32(mx) * c2;
      const bool raise = mx > m_run + kLazy;
      if (__builtin_expect(__ballot(raise) != 0, 0)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 when m_run = -inf
        l_run *= alpha;
        if constexpr (kLse) l_lse *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
      }
      if (knorm) {
        // largest key-norm bound b with qn_c2 * b <= m_run + kSafe in every
        // row (a row with q = 0 allows any; one with no max yet, none)
        const float lim = qn_c2 > 0.f ? (m_run + kSafe) / qn_c2 : __builtin_huge_valf();
        // non-negative floats order as their bits; shifted by one so that
        // "none" (-1) is the unsigned minimum
        const uint32_t u = lim >= 0.f ? (__float_as_uint(lim) >> 16) + 1u : 0u;  // bf16 bits, rounded down
        kn_lim = __builtin_amdgcn_readfirstlane(int(wave_umin(u)) - 1);
      }
    }
    fused(slot, sc, sn);  // S(i+1) is speculative when step i+1 starts a new tile
    if (!pipe) {
      finish_tile();
      if (!s1.valid) return false;
      start_tile(s1);
      qk(slot ^ 1, sn);
    }
    s0 = s1;
    s1 = cur;
    advance();
    return true;
  };
  while (iteration(0, sa, sb) && iteration(1, sb, sa)) {
  }
  wg_stamp(1);
}

__global__ void queue_reset_kernel(int* counters, int n) {
  if ((int)threadIdx.x < n) counters[threadIdx.x] = 0;
}

template <typename T, int D, int B>
hipError_t launch_t(const PrefillParams& p, int grid, hipStream_t stream) {
  if (p.lse) hipLaunchKernelGGL((prefill_kernel<T, D, B, true>), dim3(grid), dim3(2 * B), 0, stream, p);
  else hipLaunchKernelGGL((prefill_kernel<T, D, B, false>), dim3(grid), dim3(2 * B), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int D, int B, int variant, int grid,
                          hipStream_t stream) {
  if (p.queue) {
    // a kernel, not a memset, so that the call can be captured in a graph
    if (p.n_queues < 1 || p.n_queues > PrefillParams::kMaxQueues) return hipErrorInvalidValue;
    hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, stream, p.queue, p.n_queues);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dtype == 0 && B == 128 && variant == 1) return launch_prefill_wide(p, D, grid, stream);
  if (dtype == 0) {
    if (D == 128 && B == 128) return launch_t<bf16_t, 128, 128>(p, grid, stream);
    if (D == 128 && B == 64) return launch_t<bf16_t, 128, 64>(p, grid, stream);
    if (D == 64 && B == 128) return launch_t<bf16_t, 64, 128>(p, grid, stream);
    if (D == 64 && B == 64) return launch_t<bf16_t, 64, 64>(p, grid, stream);
  } else {
    if (D == 128 && B == 64) return launch_t<float, 128, 64>(p, grid, stream);
    if (D == 64 && B == 64) return launch_t<float, 64, 64>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
