// Block-sparse causal prefill attention for gfx950 with 64 query rows per wave
// (bf16 inputs, 128-row tiles).
//
// The same computation as prefill_kernel (sa_prefill.hip): exact softmax
// attention of every query row over the keys of the key blocks its (head, query
// block) tile selected, flash-style ("S-HPLB: Efficient LLM Attention Serving
// via Sparsity-Aware Head Parallelism Load Balance", Italian summary §1-2 /
// Chinese summary §1-2), in the order of the same persistent work queue or
// bins (sa_prefill_sched.hpp).  What differs is the shape of the work:
//
//   workgroup = 2 waves on one 128-row tile, two workgroups per CU: one wave
//               per SIMD, with the whole register file (O^T in the
//               accumulation registers);
//   wave      = 64 query rows, as two 32-row halves A and B;
//   step      = 32 keys of one selected key block.
// Every K fragment read from LDS feeds the Q K^T MFMAs of both halves and
// every V^T fragment the P V MFMAs of both halves, so a wave reads half the LDS
// bytes per MFMA of a 32-row wave.  32-key steps keep a half's scores in one
// 32x32 accumulator tile, which is what lets S, P and Q fit the 256 registers
// the VALU can address while O sits in the accumulation registers.
//
// One wave per SIMD leaves no other wave to fill a phase without MFMA work, so
// the softmax is split between the two MFMA phases of a step:
//   phase X(i): S(i+1) = K(i+1) Q^T for A and B   ||  softmax of S_B(i) -> P_B(i)
//   phase Y(i): O += P(i) V(i) for A and B        ||  softmax of S_A(i+1) -> P_A(i+1)
// (16 MFMAs each at D = 128).  The running maximum of a half is raised lazily
// (only when a score beats it by more than 2^kLazy, decided per half and
// wave): B's at the start of X(i), with O_B rescaled at once; A's at the start
// of Y(i), with O_A rescaled at the start of X(i+1), after P_A(i) -- still on
// the old maximum -- has been accumulated.  The normaliser sums the
// probabilities as rounded to bf16 for the P V MFMAs.
//
// Layouts as in prefill_kernel: key rows stored in LDS with bits 2 and 3 of the
// key index swapped, so the S^T accumulators are the B operand of O^T += V^T
// P^T; V^T fragments by ds_read_b64_tr_b16.  K and V are gathered through the
// block table straight into four-slot LDS rings, three steps ahead.
//
// All MFMAs are issued from inline assembly: Q K^T with Q^T in the
// accumulation registers (AGPRs) as the B operand and S^T in VGPRs, P V with
// O^T in AGPRs.  (The compiler selects AGPR forms for every builtin MFMA of a
// function that may use more than 256 registers, which would put the scores
// the softmax reads there too.)  The compiler neither sees these instructions
// as MFMAs nor inserts the wait states it would insert around them, so the
// kernel does: the step is laid out in fixed chunks separated by scheduling
// barriers, and an explicit pause (s_nop, more wait states than the 8-pass MFMA
// needs) separates an MFMA that writes S or O from a VALU access to that
// register, and a VALU write of Q or O from an MFMA that reads it.  The B
// operand P is written by the VALU at least one phase before its MFMAs.

#include "sa_device.hpp"
#include "sa_kernels.hpp"
#include "sa_prefill_common.hpp"
#include "sa_prefill_sched.hpp"

namespace sa {

namespace {

using namespace prefill;

constexpr int kWKS = 32;  // keys per step
constexpr int kWSlots = 4;  // LDS ring slots per tensor

template <int D, bool kLse>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_wide_kernel(PrefillParams p) {
  using C = Cfg<bf16_t, D, 128>;  // row layout and swizzles
  constexpr int B = 128;
  constexpr int kW = 2;                          // waves per workgroup, 64 query rows each
  constexpr int kNSub = B / kWKS;                // steps per key block
  constexpr int kTile = kWKS * C::kRow;          // bytes of one K (or V) step
  constexpr int kIPW = kTile / 1024 / kW;        // direct loads per wave and tensor per step
  constexpr int kDG = C::kDG, kDT = C::kDT;
  static_assert(kIPW * kW * 1024 == kTile, "direct loads must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char smem[2 * kWSlots * kTile];
  __shared__ QueueLds qlds;
  char* const kring = smem;                    // K slots 0..3
  char* const vring = smem + kWSlots * kTile;  // V slots 0..3

  wg_stamp(0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;   // MFMA column (query) / A-row (key, d) index
  const int half = lane >> 5;  // MFMA k-half

  Cursor<kNSub> cs;
  cs.begin(&qlds, wave, lane);
  const int S = p.S;
  const float c2 = p.scale_log2;
  const int krs = int(p.ks2 * 2);
  const int vrs = int(p.vs2 * 2);

  // ---------------------------------------------------------------- direct loads
  // Wave instruction t of a step fills LDS bytes [1024 t, 1024 t + 1024): lane i
  // writes 16 bytes at 1024 t + 16 i, i.e. LDS row r = (1024 t + 16 i) / kRow,
  // physical chunk cp; it fetches the global row and chunk the swizzle puts there.
  int k_voff[kIPW], v_voff[kIPW];
#pragma unroll
  for (int u = 0; u < kIPW; ++u) {
    const int t = wave * kIPW + u;
    const int byte = t * 1024 + lane * 16;
    const int r = byte / C::kRow, cp = (byte % C::kRow) / 16;
    k_voff[u] = perm_key(r) * krs + (cp ^ C::swz_k(r)) * 16;
    v_voff[u] = r * vrs + (cp ^ C::swz_v(r)) * 16;
  }
  // The buffer starts at the step's first key row and ends at the sequence
  // end, so rows past the end read as zero and the per-lane offsets stay fixed.
  // Returns the number of loads issued by this wave.
  auto fetch = [&](const Step& s, int slot, bool k_side) __attribute__((always_inline)) -> int {
    if (!s.valid) return 0;
    const int kb = s.kvs >> 16, kh = s.kvs & 0xffff;
    const char* base = k_side ? reinterpret_cast<const char*>(p.k) + (kb * p.ks0 + kh * p.ks1) * (int64_t)2
                              : reinterpret_cast<const char*>(p.v) + (kb * p.vs0 + kh * p.vs1) * (int64_t)2;
    const int rs = k_side ? krs : vrs;
    const int row = s.n * B + s.hs * kWKS;
    const i32x4 r = buffer_rsrc_words(base + (int64_t)row * rs, max(S - row, 0) * rs);
    char* dst = (k_side ? kring : vring) + slot * kTile + wave * kIPW * 1024;
#pragma unroll
    for (int u = 0; u < kIPW; ++u) dma16_async(r, dst + u * 1024, k_side ? k_voff[u] : v_voff[u]);
    return kIPW;
  };

  // ---------------------------------------------------------------- tile state
  // Half A: query rows 64 wave + col, half B: 64 wave + 32 + col of the tile.
  u32x4 qa[kDG], qb[kDG];   // Q^T fragments
  f32x16 oa[kDT], ob[kDT];  // O^T accumulators (AGPRs)
  // running max (log2 domain), sum of the bf16-rounded probabilities (the
  // normaliser), sum of the unrounded ones (lse only)
  float ma = kNegInf, mb = kNegInf, la = 0.f, lb = 0.f, xa = 0.f, xb = 0.f;
  int t_bh = 0, t_m = 0;

  // O^T += V^T P^T (the builtin: a function that may use more than 256
  // registers gets the AGPR form, so O^T lives in the accumulation registers,
  // and the compiler knows this instruction's latency for every access to O)
  auto mfma_o = [](f32x16& acc, u32x4 a, u32x4 b) __attribute__((always_inline)) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                  0, 0, 0);
  };
  // S^T = K Q^T (first d group: C = 0, then accumulate), Q^T in AGPRs
  auto mfma_s0 = [](f32x16& acc, u32x4 a, u32x4 b) __attribute__((always_inline)) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "a"(b));
  };
  auto mfma_s = [](f32x16& acc, u32x4 a, u32x4 b) __attribute__((always_inline)) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
  };
  // Wait states between an MFMA and a VALU access to its result, or a VALU
  // write and an MFMA that reads it (24: more than the passes of
  // v_mfma_f32_32x32x16_bf16 plus the extra states its result needs).
  auto pause = []() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
  // Makes the accumulation registers the home of a value (Q^T, O^T): defined
  // there by an asm output, it is not copied back for its MFMA operands.
  auto to_agpr = [](auto& x) __attribute__((always_inline)) { asm("" : "+a"(x)); };

  // Q^T fragments of the tile of step s (into the accumulation registers)
  auto load_q = [&](const Step& s) __attribute__((always_inline)) {
    const int Hq = COLD(Hq);
    const int bi = s.bh / Hq, h = s.bh % Hq;
    const int qrow = s.m * B + wave * 64 + col;
    const char* rp = reinterpret_cast<const char*>(COLD(q)) +
                     (bi * COLD(qs0) + h * COLD(qs1) + (int64_t)qrow * COLD(qs2)) * (int64_t)2;
    const int64_t rstep = 32 * COLD(qs2) * (int64_t)2;
#pragma unroll
    for (int dg = 0; dg < kDG; ++dg) {
      // lane half g holds d = 16 dg + 8 g .. +7
      const int d0 = dg * 16 + half * 8;
      qa[dg] = qrow < S ? *reinterpret_cast<const u32x4*>(rp + d0 * 2) : u32x4{0u, 0u, 0u, 0u};
      qb[dg] = qrow + 32 < S ? *reinterpret_cast<const u32x4*>(rp + rstep + d0 * 2) : u32x4{0u, 0u, 0u, 0u};
      to_agpr(qa[dg]);
      to_agpr(qb[dg]);
    }
    pause();  // before an MFMA reads them
  };
  auto zero_o = [&]() __attribute__((always_inline)) {
    pause();  // the last MFMAs are done with O
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      oa[dt] = f32x16{};
      ob[dt] = f32x16{};
    }
    fence();
  };

  auto finish_half = [&](const f32x16 (&o)[kDT], float l_w, float l_x, float m, int row_off) {
    const int Hq = COLD(Hq);
    const int bi = t_bh / Hq, h = t_bh % Hq;
    const float l = sum_xor32(l_w);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lx = kLse ? sum_xor32(l_x) : l;
    const int qrow = t_m * B + wave * 64 + row_off + col;
    if (qrow < S) {
      const int64_t orow = bi * COLD(os0) + h * COLD(os1) + (int64_t)qrow * COLD(os2);
      void* const out = COLD(o);
      const bool out_f32 = COLD(out_f32);
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        fence();  // one accumulator tile at a time in VGPRs
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = dt * 32 + r4 * 8 + half * 4;
          const float o0 = o[dt][r4 * 4 + 0] * inv, o1 = o[dt][r4 * 4 + 1] * inv;
          const float o2 = o[dt][r4 * 4 + 2] * inv, o3 = o[dt][r4 * 4 + 3] * inv;
          if (!out_f32) {
            *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(out) + orow + d) =
                uint2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + orow + d) = f32x4{o0, o1, o2, o3};
          }
        }
      }
      float* const lse = COLD(lse);
      if (kLse && half == 0) lse[(int64_t)t_bh * S + qrow] = lx > 0.f ? (m + __log2f(lx)) * kLn2 : kNegInf;
    }
  };
  auto finish_tile = [&](float la_, float xa_, float ma_, float lb_, float xb_, float mb_) __attribute__((always_inline)) {
    pause();  // the last MFMAs are done with O
    finish_half(oa, la_, xa_, ma_, 0);
    finish_half(ob, lb_, xb_, mb_, 32);
  };

  // ---------------------------------------------------------------- pieces of a step
  // K fragment (d group dg) of K slot ks
  auto kfrag = [&](const char* ks, int dg) __attribute__((always_inline)) {
    return lds16(ks, col * C::kRow + ((dg * 2 + half) ^ C::swz_k(col)) * 16);
  };
  // V^T fragment (key chunk kc, d tile dt) of V slot vs: 16-lane group G
  // covers d = 32 dt + 16 (G % 2) + lane % 16 and keys 16 kc + 8 (G / 2) +
  // 4 r + 0..3; source lane j of the group points at V row k0 + j / 4,
  // columns dbase + 4 (j % 4) .. +3.
  auto vfrag = [&](const char* vs, int kc, int dt) __attribute__((always_inline)) {
    const int G = lane >> 4, j = lane & 15;
    const int d = dt * 32 + (G & 1) * 16 + (j & 3) * 4;
    const int row0 = kc * 16 + (G >> 1) * 8 + (j >> 2);
    const int row1 = row0 + 4;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(vs + row0 * C::kRow + (((d >> 3) ^ C::swz_v(row0)) << 4) + ((d & 7) << 1)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(vs + row1 * C::kRow + (((d >> 3) ^ C::swz_v(row1)) << 4) + ((d & 7) << 1)));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // One pair of probabilities of a half: scores i, i+1 -> packed bf16 word of
  // P^T fragment kc; the sums take the rounded values (and the unrounded ones
  // for lse).  Element i of a half's S^T tile is key 16 (i / 8) + 8 half + i % 8.
  auto prob_pair = [&](const f32x16& sc, int pair, float mu, u32x4 (&pf)[2], float& s0, float& s1, float& x0,
                       float& x1) {
    const int kc = pair >> 2, w = pair & 3;
    const int i = kc * 8 + 2 * w;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, -mu));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i + 1], c2, -mu));
    const uint32_t pk = pack_bf16x2(p0, p1);
    pf[kc][w] = pk;
    s0 += bf16_lo(pk);
    s1 += bf16_hi(pk);
    if constexpr (kLse) {
      x0 += p0;
      x1 += p1;
    }
  };
  // Q K^T of both halves from K slot `slot`, not interleaved (tile start;
  // ends with the pause before the VALU reads S)
  auto qk_both = [&](int slot, f32x16& sa, f32x16& sb) __attribute__((always_inline)) {
    const char* ks = kring + slot * kTile;
    pause();  // Q was just written
#pragma unroll
    for (int dg = 0; dg < kDG; ++dg) {
      const u32x4 a = kfrag(ks, dg);
      if (dg == 0) {
        mfma_s0(sa, a, qa[dg]);
        mfma_s0(sb, a, qb[dg]);
      } else {
        mfma_s(sa, a, qa[dg]);
        mfma_s(sb, a, qb[dg]);
      }
    }
    pause();
  };
  // whole softmax of a half, not interleaved (tile start)
  auto softmax_half = [&](const f32x16& sc, u32x4 (&pf)[2], float m, float& l, float& x) {
    const float mu = m == kNegInf ? 0.f : m;
    float s0 = 0.f, s1 = 0.f, x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int pair = 0; pair < 8; ++pair) prob_pair(sc, pair, mu, pf, s0, s1, x0, x1);
    l += s0 + s1;
    if constexpr (kLse) x += x0 + x1;
  };
  // Masking of a half's scores of step s in place (causal diagonal, sequence
  // tail), when any key of the step is invisible to a row of the half.
  auto mask_half = [&](const Step& s, f32x16& sc, int row_off) __attribute__((always_inline)) {
    const int key0 = s.hs * kWKS;
    const int q0 = wave * 64 + row_off;  // first query row of the half in the tile
    if (!((s.n == s.m && key0 + kWKS - 1 > q0) || s.n * B + key0 + kWKS > S)) return;
    const bool diag = s.n == s.m;
    const int lim = min(diag ? q0 + col : B, S - s.n * B - 1);  // largest visible key of the block
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = key0 + (i >> 3) * 16 + half * 8 + (i & 7);
      sc[i] = kl > lim ? kNegInf : sc[i];
    }
  };
  // Row max of a half's step; raises m when it beats it by more than 2^kLazy.
  // alpha: the per-row factor that brings earlier sums to the new maximum (1
  // when not raised, 0 when raised from -inf).  Returns whether any row raised.
  auto raise_max = [&](const f32x16& sc, float& m, float& alpha) __attribute__((always_inline)) -> bool {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, sc[i]), sc[i + 1]);
    mx = max_xor32(mx) * c2;
    const bool raise = mx > m + kLazy;
    alpha = 1.f;
    if (__builtin_expect(__ballot(raise) != 0, 0)) {
      const float m_new = raise ? mx : m;
      alpha = raise ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;  // 0 when m was -inf
      m = m_new;
      return true;
    }
    return false;
  };

  // Phase X: S(i+1) for both halves from K slot kslot, interleaved with the
  // softmax of half B of step i (sbc -> pb).  Chunk dg: the K fragment of d
  // group dg + 2 is read, and the two MFMAs of d group dg each carry half of
  // one probability pair.  Ends with the pause before the VALU reads S.
  auto phase_x = [&](int kslot, f32x16& sa, f32x16& sbn, const f32x16& sbc, u32x4 (&pb)[2]) {
    static_assert(kDG == 8 || kDG == 4, "d groups");
    constexpr int kPairs = 8 / kDG;  // probability pairs per chunk
    const char* ks = kring + kslot * kTile;
    const float mu = mb == kNegInf ? 0.f : mb;
    float s0 = 0.f, s1 = 0.f, x0 = 0.f, x1 = 0.f;
    u32x4 kf[kDG];
    kf[0] = kfrag(ks, 0);
    kf[1] = kfrag(ks, 1);
#pragma unroll
    for (int dg = 0; dg < kDG; ++dg) {
      fence();
      if (dg + 2 < kDG) kf[dg + 2] = kfrag(ks, dg + 2);
      if (dg == 0) mfma_s0(sa, kf[dg], qa[dg]);
      else mfma_s(sa, kf[dg], qa[dg]);
      prob_pair(sbc, dg * kPairs, mu, pb, s0, s1, x0, x1);
      if (dg == 0) mfma_s0(sbn, kf[dg], qb[dg]);
      else mfma_s(sbn, kf[dg], qb[dg]);
      if (kPairs > 1) prob_pair(sbc, dg * kPairs + 1, mu, pb, s0, s1, x0, x1);
    }
    fence();
    lb += s0 + s1;
    if constexpr (kLse) xb += x0 + x1;
    pause();
  };
  // Phase Y: O += P(i) V(i) for both halves from V slot vslot, interleaved with
  // the softmax of half A of step i+1 (sa -> pan).  Chunk (kc, dt): the V^T
  // fragment two chunks ahead is read, and the two MFMAs carry one pair (D =
  // 128) or two (D = 64).
  auto phase_y = [&](int vslot, const u32x4 (&pac)[2], const u32x4 (&pb)[2], const f32x16& sa, u32x4 (&pan)[2]) {
    constexpr int kCh = 2 * kDT;       // chunks
    constexpr int kPairs = 8 / kCh;    // probability pairs per chunk
    const char* vs = vring + vslot * kTile;
    const float mu = ma == kNegInf ? 0.f : ma;
    float s0 = 0.f, s1 = 0.f, x0 = 0.f, x1 = 0.f;
    u32x4 vf[kCh];
    vf[0] = vfrag(vs, 0, 0);
    vf[1] = vfrag(vs, 1 / kDT, 1 % kDT);
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int kc = c / kDT, dt = c % kDT;
      fence();
      if (c + 2 < kCh) vf[c + 2] = vfrag(vs, (c + 2) / kDT, (c + 2) % kDT);
      mfma_o(oa[dt], vf[c], pac[kc]);
      prob_pair(sa, c * kPairs, mu, pan, s0, s1, x0, x1);
      mfma_o(ob[dt], vf[c], pb[kc]);
      if (kPairs > 1) prob_pair(sa, c * kPairs + 1, mu, pan, s0, s1, x0, x1);
    }
    fence();
    la += s0 + s1;
    if constexpr (kLse) xa += x0 + x1;
  };

  // ---------------------------------------------------------------- walk
  // s0 = step i (its P V this iteration), s1 = i+1 (its Q K^T), s2, s3, and
  // cs.cur = i+4.  Step j's K and V sit in slot j % 4; iteration i fetches
  // K(i+4) and V(i+3), so at its start K(i+1) and V(i) (fetched three
  // iterations earlier) must have landed while the loads of the last two
  // iterations may stay in flight.
  Step s0 = cs.cur;
  if (!s0.valid) {
    wg_stamp(1);
    return;
  }
  cs.advance();
  Step s1 = cs.cur;
  cs.advance();
  Step s2 = cs.cur;
  cs.advance();
  Step s3 = cs.cur;
  cs.advance();
  // the loads of virtual iterations -4 .. -1
  fetch(s0, 0, true);
  fetch(s1, 1, true);
  fetch(s0, 0, false);
  int n_prev2 = fetch(s2, 2, true) + fetch(s1, 1, false);  // iteration -2
  int n_prev1 = fetch(s3, 3, true) + fetch(s2, 2, false);  // iteration -1
  auto wait_ready = [&](int in_flight) __attribute__((always_inline)) {
    // in_flight: a multiple of kIPW, at most 4 kIPW (two iterations of K and V)
    if (in_flight >= 4 * kIPW) wait_vmcnt<4 * kIPW>();
    else if (in_flight >= 3 * kIPW) wait_vmcnt<3 * kIPW>();
    else if (in_flight >= 2 * kIPW) wait_vmcnt<2 * kIPW>();
    else if (in_flight >= kIPW) wait_vmcnt<kIPW>();
    else wait_vmcnt<0>();
  };
  wait_vmcnt<0>();
  __syncthreads();

  f32x16 sA, sB0, sB1;
  u32x4 pA0[2], pA1[2], pB[2];
  // factors still owed by O_A (raised at the start of the last Y phase) and
  // O_B; both 0 after a tile change, which is how O is cleared for the next
  // tile
  float alpha_a = 1.f;
  bool pend_a = false, clear_b = false;

  // the first tile: Q, S(0) for both halves, half A's maximum and probabilities
  t_bh = s0.bh;
  t_m = s0.m;
  load_q(s0);
  zero_o();
  qk_both(0, sA, sB0);
  mask_half(s0, sA, 0);
  {
    float a;
    raise_max(sA, ma, a);  // from -inf: la is still zero
  }
  softmax_half(sA, pA0, ma, la, xa);

  // One step.  A tile change (step i+1 starts another tile, or there is no
  // step i+1) runs through the same phases: the next tile's Q is loaded before
  // phase X (the current Q's last use, Q K^T of step i, was in the previous
  // iteration), so S(i+1) is the new tile's; after phase X the finishing
  // tile's maxima and sums are set aside and reset; after phase Y, which still
  // accumulates the finishing tile's P(i) V(i), its output is written, and the
  // next iteration's rescale clears O (factor 0).  After the last step the
  // phases run once more on stale data that nothing uses.
  auto iteration = [&](int i4, f32x16& sbc, f32x16& sbn, u32x4 (&pac)[2], u32x4 (&pan)[2])
                       __attribute__((always_inline)) -> bool {
    // i4 = i % 4: K(i+1) is in slot (i4 + 1) % 4, V(i) in slot i4
    wait_ready(n_prev2 + n_prev1);
    __syncthreads();  // also: every wave is done with the slots refilled here
    const int n_now = fetch(cs.cur, i4, true) + fetch(s3, (i4 + 3) & 3, false);  // K(i+4), V(i+3)
    n_prev2 = n_prev1;
    n_prev1 = n_now;
    // half B of step i: mask, maximum; O_A's pending factor and O_B's together
    mask_half(s0, sbc, 32);
    float alpha_b;
    const bool raised_b = raise_max(sbc, mb, alpha_b);
    lb *= alpha_b;
    if constexpr (kLse) xb *= alpha_b;
    if (__builtin_expect(raised_b || pend_a || clear_b, 0)) {
      const float fb = clear_b ? 0.f : alpha_b;
      pause();
      // one accumulator tile at a time through the VGPRs
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) {
        oa[dt] *= alpha_a;
        ob[dt] *= fb;
      }
      pause();
    }
    pend_a = false;
    clear_b = false;
    alpha_a = 1.f;
    const bool change = !s1.valid || s1.item != s0.item;
    if (__builtin_expect(change && s1.valid, 0)) load_q(s1);
    phase_x((i4 + 1) & 3, sA, sbn, sbc, pB);
    float fla = 0.f, fxa = 0.f, fma_ = 0.f, flb = 0.f, fxb = 0.f, fmb = 0.f;
    if (__builtin_expect(change, 0)) {
      fla = la, fxa = xa, fma_ = ma, flb = lb, fxb = xb, fmb = mb;
      ma = mb = kNegInf;
      la = lb = xa = xb = 0.f;
      alpha_a = 0.f;
      pend_a = true;
      clear_b = true;
    }
    // half A of step i+1: mask and maximum; O_A is rescaled after this
    // phase's P V, which still accumulates P_A(i) on the old maximum
    mask_half(s1, sA, 0);
    {
      float a;
      if (__builtin_expect(raise_max(sA, ma, a), 0)) {
        la *= a;
        if constexpr (kLse) xa *= a;
        if (!change) alpha_a = a;
        pend_a = true;
      }
    }
    phase_y(i4, pac, pB, sA, pan);
    if (__builtin_expect(change, 0)) {
      finish_tile(fla, fxa, fma_, flb, fxb, fmb);
      if (!s1.valid) return false;
      t_bh = s1.bh;
      t_m = s1.m;
    }
    s0 = s1;
    s1 = s2;
    s2 = s3;
    s3 = cs.cur;
    cs.advance();
    return true;
  };
  while (iteration(0, sB0, sB1, pA0, pA1) && iteration(1, sB1, sB0, pA1, pA0) &&
         iteration(2, sB0, sB1, pA0, pA1) && iteration(3, sB1, sB0, pA1, pA0)) {
  }
  wait_vmcnt<0>();  // no load may still write LDS when the workgroup ends
  wg_stamp(1);
}

template <int D>
hipError_t launch_d(const PrefillParams& p, int grid, hipStream_t stream) {
  if (p.lse) hipLaunchKernelGGL((prefill_wide_kernel<D, true>), dim3(grid), dim3(128), 0, stream, p);
  else hipLaunchKernelGGL((prefill_wide_kernel<D, false>), dim3(grid), dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_wide(const PrefillParams& p, int D, int grid, hipStream_t stream) {
  if (D == 128) return launch_d<128>(p, grid, stream);
  if (D == 64) return launch_d<64>(p, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
