// Launch interfaces of the gfx950 kernels (host side).  Only sa_api.cpp calls
// these, after validating every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kMaxHeads = 128;

// Per-head budget parameters, passed by value in kernel arguments.
struct HeadTable {
  int32_t min_blocks[kMaxHeads];
  uint32_t ratio_q16[kMaxHeads];
  int16_t n_sink[kMaxHeads];
  int16_t n_local[kMaxHeads];
  int16_t gran[kMaxHeads];
};

// ---------------------------------------------------------------- pooling
// Paged KV: each KV head has its own pool of physical pages of page_size
// token rows; page_table[(b * heads + h) * max_pages + p] is the physical page
// (in head h's pool) of logical page p of sequence b.
struct PageTable {
  const int32_t* table = nullptr;  // nullptr: contiguous cache
  int page_size = 0, max_pages = 0, pages_per_head = 0;
};

struct PoolParams {
  const void* x;         // [batch][heads][T][D] (strided); paged: pools at x + h * s1, rows s2 apart
  int64_t s0, s1, s2;    // strides in elements
  float* out;            // [batch][heads][nb][D] fp32, contiguous
  int heads, T, g, nb, blocks_per_wg;
  PageTable pages;       // g divides page_size
  // nullable: [batch][heads][nb] fp32, the largest Euclidean norm of a row of
  // each block (contiguous rows only, not with pages)
  float* norm_max = nullptr;
};
hipError_t launch_pool(const PoolParams& p, int dtype, int D, int batch, hipStream_t stream);

// ---------------------------------------------------------------- prefill selection
// Pool + score + top-k in one kernel: a workgroup takes up to kSelRows
// consecutive query blocks of one (sequence, query head); their scores against
// the causal pooled keys live in LDS, rows padded to sel_rowlen floats.
constexpr int kSelRows = 16;
constexpr int kSelFloats = kSelRows * (1024 + 32 + 4);
constexpr int kSelMaxBlocks = 8192;
__host__ __device__ inline int sel_rowlen(int nb) {
  const int nbp = (nb + 63) & ~63;
  return nbp + nbp / 32 + 4;  // one pad float per 32 (top-k reads), + 4 (MFMA row stores)
}
__host__ __device__ inline int sel_rows(int nb) {
  const int r = kSelFloats / sel_rowlen(nb);
  return r < kSelRows ? r : kSelRows;
}
struct PrefillSelectParams {
  const void* q;      // [batch][Hq][S][D] (strided, D contiguous), dtype bf16 or fp32
  int64_t qs0, qs1, qs2;
  const float* kp;    // pooled keys [batch*Hkv][NB][D]
  int32_t* idx;       // out: [batch*Hq*NB][kmax]
  int32_t* cnt;       // out: [batch*Hq*NB]
  int kmax;
  int Hq, G, S, NB;
  int R, rowlen, n_mg;  // rows per workgroup, LDS row length, workgroups per (sequence, head)
  float scale;
  HeadTable heads;
};
// grid: batch * Hq * n_mg workgroups of 256 threads; block 64 or 128, D 64 or 128
hipError_t launch_select_prefill(const PrefillSelectParams& p, int dtype, int D, int block, int batch,
                                 hipStream_t stream);

struct TopkParams {
  const float* s;       // scores; row r at s + r * s_row
  int64_t s_row;
  int32_t* idx;         // out: row r at idx + r * kmax
  int32_t* cnt;         // out: [rows]
  int kmax;
  int rows;
  int Hq;               // rows (b, h) = b * Hq + h
  int kv_len;
  HeadTable heads;
};
hipError_t launch_topk(const TopkParams& p, int max_cand, hipStream_t stream);

// ---------------------------------------------------------------- decode selection
struct DecodeScoreJob {
  int kvh;        // KV head
  int pool;       // index of the pooled array (granularity class)
  int n_heads;
  int heads[8];
};
constexpr int kMaxScoreJobs = 48;
struct DecodeScoreParams {
  const void* q;          // [batch][Hq][D]
  int64_t qs0, qs1;
  const float* pooled;    // concatenated pooled arrays
  int64_t pool_off[4];    // element offset of each pooled array
  int pool_nc[4];         // blocks per head of each pooled array
  float* s;               // [batch][Hq][nc_max]
  int nc_max, Hq, Hkv, n_jobs, rows_per_wg;
  float scale;
  DecodeScoreJob jobs[kMaxScoreJobs];
};
hipError_t launch_decode_scores(const DecodeScoreParams& p, int dtype, int D, int batch, hipStream_t stream);

// ---------------------------------------------------------------- prefill attention
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  const int32_t* block_idx;
  const int32_t* block_cnt;
  int kmax;
  const int32_t* bin_offsets;   // nullable
  const int32_t* items_by_bin;
  int Hq, G, S, NB, n_tiles;
  float scale_log2;
  int out_f32;
  int* queue;  // work-queue counters (nullable): items_by_bin is then one global order
  // Work-queue partitions: positions [qoff[i], qoff[i+1]) of items_by_bin form
  // queue i, counted by queue[i]; workgroup w starts on queue w % n_queues and
  // moves to the next queue when its own is empty.  One queue: n_queues = 1,
  // qoff = {0, n_tiles}.
  static constexpr int kMaxQueues = 16;
  int n_queues = 1;
  int qoff[kMaxQueues + 1] = {};
  // nullable: workgroup w writes the constant clock (s_memrealtime) at its
  // start to wg_times[2 w] and at its end to wg_times[2 w + 1]
  uint64_t* wg_times = nullptr;
  // nullable: [batch][Hkv][NB] fp32, an upper bound of the Euclidean norm of
  // every key row of each key block (PoolParams::norm_max); lets the kernel
  // skip the running-max check of steps whose scores cannot overflow
  const float* key_norms = nullptr;
};
// grid = persistent bins, queue workers or tiles.  variant 0: the
// 32-rows-per-wave kernel (B/32 waves); variant 1 (bf16, B = 128): the
// 64-rows-per-wave kernel (workgroups of 2 waves).
hipError_t launch_prefill(const PrefillParams& p, int dtype, int D, int B, int variant, int grid,
                          hipStream_t stream);
hipError_t launch_prefill_wide(const PrefillParams& p, int D, int grid, hipStream_t stream);

// ---------------------------------------------------------------- decode attention
// Union of the selected 16-token atoms of the query heads of one KV group.
constexpr int kAtom = 16;
struct DecodePlanParams {
  const int32_t* block_idx;  // [batch][Hq][kmax]
  const int32_t* block_cnt;  // [batch][Hq]
  int kmax, Hq, Hkv, G, kv_len, n_atoms;  // n_atoms = ceil(kv_len / 16)
  int max_union;             // capacity of the atom list per (b, kvh)
  uint32_t* atoms;           // out: [batch][Hkv][max_union]: atom index | head mask << 24
  int32_t* n_union;          // out: [batch][Hkv]
  HeadTable heads;
};
hipError_t launch_decode_plan(const DecodePlanParams& p, int batch, hipStream_t stream);

// Per chunk partial of one head: running max (log2 domain), the sum of the
// probabilities as they weighted the V rows (bf16-rounded for bf16 inputs: the
// normaliser of o), and the same sum before rounding (for lse).
constexpr int kPartMl = 3;
struct DecodeAttnParams {
  const void* q;
  int64_t qs0, qs1;
  const void* k;
  const void* v;
  int64_t ks0, ks1, ks2, vs0, vs1, vs2;
  const uint32_t* atoms;
  const int32_t* n_union;
  int max_union, chunk_atoms, n_chunks;  // chunks per (b, kvh)
  int Hq, Hkv, G, kv_len;
  float scale_log2;
  PageTable pages;  // paged: k, v are the pools (head stride ks1 / vs1, row stride ks2 / vs2)
  float* part_o;    // [batch][Hkv][n_chunks][G][D]
  float* part_ml;   // [batch][Hkv][n_chunks][G][kPartMl]
};
hipError_t launch_decode_attn(const DecodeAttnParams& p, int dtype, int D, int batch, hipStream_t stream);

struct DecodeCombineParams {
  const float* part_o;
  const float* part_ml;
  const int32_t* n_union;
  int chunk_atoms, n_chunks, Hq, Hkv, G;
  void* o;
  int64_t os0, os1;
  float* lse;
  int out_f32;
};
hipError_t launch_decode_combine(const DecodeCombineParams& p, int dtype, int D, int batch, hipStream_t stream);

// ---------------------------------------------------------------- calibration
struct MassParams {
  const void* q;  // bf16 [batch][Hq][S][D] (strided)
  const void* k;  // bf16 [batch][Hkv][S][D] (strided)
  int64_t qs0, qs1, qs2, ks0, ks1, ks2;
  float* mass;    // [batch][Hq][NB][NB] fp32
  int Hq, G, S, NB;
  float scale_log2;
};
// block size 128; D 64 or 128
hipError_t launch_block_mass(const MassParams& p, int D, int batch, hipStream_t stream);

struct DeviationParams {
  const float* a;  // fp32 [batch][Hq][S][D] (strided, D contiguous)
  const float* r;  // same layout
  int64_t s0, s1, s2;
  int batch, Hq, S, D;
  double* dev;     // [Hq]
};
// one workgroup per query head
hipError_t launch_output_deviation(const DeviationParams& p, hipStream_t stream);


// roofline denominators: 8 independent chains of 32x32x16 bf16 MFMAs per wave
// (four waves per workgroup), and a grid-stride non-temporal read of a buffer
hipError_t launch_mfma_peak(int n_workgroups, int iters, bool random_operands, float* sink, hipStream_t stream);
hipError_t launch_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int n_workgroups, hipStream_t stream);

}  // namespace sa
