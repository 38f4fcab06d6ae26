/*
 * sparse_attn.h -- C ABI of the per-head heterogeneous block-sparse attention
 * library for AMD MI355X (gfx950).  libsparse_attn.so exports exactly the
 * functions declared here.
 *
 * The operations (gist.science technical summaries):
 *   - select_blocks: mean-pool keys (and query blocks) into blocks, score every
 *     (head, query block) against the pooled keys and keep a per-head budget of
 *     top-scoring key blocks, sink and local blocks always kept.  Per-head
 *     budgets: "S-HPLB: Efficient LLM Attention Serving via Sparsity-Aware Head
 *     Parallelism Load Balance", Italian summary §2.A and Chinese summary §2.1;
 *     top-k sparse attention: same pages §1; block granularity and
 *     streaming/retrieval heads: "Fluxion", Italian summary, Intuizioni Chiave
 *     1-2; Index/Select operations: "Unifying Sparse Attention with
 *     Hierarchical Memory for Scalable Long-Context LLM Serving" (Spin),
 *     Spanish summary §2.A.
 *   - lpt_schedule: greedy longest-load-first placement of work items on bins
 *     (S-HPLB, Italian summary §2.B, Chinese summary §2.2).  On one GPU the
 *     items are (head, query-block) tiles and the bins are the persistent
 *     workgroups of the prefill kernel.
 *   - sparse_attn_prefill / sparse_attn_decode: exact softmax attention of every
 *     query over the keys of its selected blocks only (causal for prefill), with
 *     grouped-query (GQA) heads sharing one KV head ("Fluxion", Componenti di
 *     Sistema: GQA handled at KV-group level).
 *
 * Conventions
 *   - "[dev]" pointers are HIP device memory owned by the caller; "[host]"
 *     pointers are host memory owned by the caller.  The library never
 *     allocates or frees caller-visible memory; scratch space is the caller's
 *     workspace, sized by the *_workspace_size functions.
 *   - Tensors are addressed as base + b*stride[0] + h*stride[1] + t*stride[2] + d
 *     (strides in elements; the head_dim axis is contiguous).
 *   - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns after enqueueing.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - Every function validates all arguments before enqueueing anything: on
 *     error nothing is launched, a negative sa_status is returned and
 *     sa_last_error() describes it.
 *   - Thread safety: calls are reentrant; the error text is per thread.  Calls
 *     that share a workspace must be ordered on one stream.
 *   - Q, K and V must be finite (no NaN or infinity); results are unspecified
 *     otherwise.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sa_status;
enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1, /* bad shape, pointer, budget or size */
  SA_ERR_UNSUPPORTED = -2, /* valid but not implemented (head_dim, block, dtype, limits) */
  SA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than *_workspace_size */
  SA_ERR_HIP = -4,         /* a HIP runtime call failed (name in sa_last_error) */
  SA_ERR_NO_DEVICE = -5,   /* no HIP device visible */
  SA_ERR_ARCH = -6         /* current device is not gfx950 */
};

enum { SA_BF16 = 0, SA_F32 = 1 };

#define SA_MAX_HEADS 128

/* Shape of one attention call.
 *   prefill: q_len == kv_len (causal self-attention, both start at token 0);
 *            block_size is the query/key block (64 or 128).
 *   decode:  q_len == 1; the query is the token at position kv_len-1 and sees
 *            all kv_len cached tokens; block_size is ignored (each head has its
 *            own granularity in sa_head_budget).
 * head_dim: 64 or 128.  dtype: SA_BF16 or SA_F32 for Q/K/V.
 * softmax_scale: 0 means 1/sqrt(head_dim).  kernel_variant: see the field.
 * Strides: prefill q/o [batch][n_q_heads][q_len][head_dim], k/v
 * [batch][n_kv_heads][kv_len][head_dim]; decode q/o use stride[2] unused
 * ([batch][n_q_heads][head_dim]). */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t q_len, kv_len;
  int32_t block_size;
  int32_t dtype;
  float softmax_scale;
  int32_t kernel_variant; /* prefill attention: 0 = 32 query rows per wave (default), 1 = 64
                             query rows per wave (bf16 with block_size 128; others run 0);
                             same results up to rounding order */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
} sa_attn_desc;

/* Budget of one query head (one entry per query head, [host]).
 * A row with n candidate blocks keeps
 *   k = min(n, max(min_blocks, ceil(ratio_q16 * n / 65536)))
 * blocks (exact integer arithmetic): the first n_sink and last n_local
 * candidates always, the rest by descending score, ties to the lower block
 * index.  Candidates: prefill row m sees blocks 0..m; a decode head sees
 * ceil(kv_len / granularity) blocks.  Requires 1 <= min_blocks and
 * n_sink + n_local <= min_blocks.  granularity: decode tokens per block
 * (16, 32, 64 or 128; ignored in prefill). */
typedef struct {
  int32_t min_blocks;
  uint32_t ratio_q16;
  int32_t n_sink, n_local;
  int32_t granularity;
} sa_head_budget;

int32_t sa_version(void);
/* Text of the last error on the calling thread ("" if none).  Valid until the
 * next call on this thread. */
const char* sa_last_error(void);

/* Host-side checks of the index tables before every attention launch:
 * block_idx / block_cnt (counts in [0, kmax]; entries strictly increasing,
 * prefill in [0, m], decode in [0, ceil(kv_len / granularity))), the prefill
 * schedule (items_by_bin a permutation of the tiles, bin offsets from 0 to the
 * tile count, non-decreasing) and, for paged decode, the page-table entries of
 * the pages in use (in [0, pages_per_head)).  A failed check returns
 * SA_ERR_INVALID_ARG with the first bad entry in sa_last_error, and nothing is
 * launched.  The checks copy the tables to the host after synchronising the
 * stream, so they are for debugging, not for the timed path.  A call on a
 * stream that is being captured into a graph skips them (a capture allows
 * neither the synchronisation nor the copies); the calls before the capture,
 * such as its warm-up, are checked.  Off by default; on when SA_DEBUG_CHECKS
 * is set (and not "0") in the environment when the library loads.  Returns the
 * previous setting; process-wide. */
int32_t sa_set_debug_checks(int32_t on);

/* ---------------------------------------------------------------- host-only */

/* Greedy longest-load-first placement (host, synchronous, O(n log n + n log
 * n_bins)).  Items are taken by load, largest first, ties to the lower item
 * index; each goes to the bin with the least load so far, ties to the lower
 * bin index.
 *   loads[n_items]           [host] non-negative
 *   bin_of_item[n_items]     [host] out: bin of each item
 *   bin_offsets[n_bins+1]    [host] out: CSR offsets into items_by_bin
 *   items_by_bin[n_items]    [host] out: items of bin b, in assignment order,
 *                            at [bin_offsets[b], bin_offsets[b+1])
 *   bin_load[n_bins]         [host] out: total load per bin (may be NULL)
 * n_items >= 0, n_bins >= 1; a negative load is SA_ERR_INVALID_ARG. */
sa_status sa_lpt_schedule(const int64_t* loads, int32_t n_items, int32_t n_bins,
                          int32_t* bin_of_item, int32_t* bin_offsets, int32_t* items_by_bin,
                          int64_t* bin_load);

/* Two-level greedy longest-load-first placement for a GPU whose compute units
 * sit in n_groups partitions with a cache of their own (8 XCDs on MI355X;
 * workgroup b of a persistent grid runs on partition b % n_groups).  Items are
 * first bundled into chunks chosen by the caller (chunk_of_item[i] in
 * [0, n_chunks)); level 1 places the chunks on the groups with
 * sa_lpt_schedule's rule (chunk load = sum of its items' loads); level 2 places
 * each group's items on that group's n_bins / n_groups bins, again with
 * sa_lpt_schedule's rule, bin b of the group being b * n_groups + group.  Items
 * of one chunk so share a partition's cache.  This adapts the S-HPLB greedy
 * placement ("S-HPLB ...", Italian summary §2.B, Chinese summary §2.2) to a
 * device with partitioned caches; on one partition it is sa_lpt_schedule.
 *   loads, chunk_of_item [host][n_items]; outputs as for sa_lpt_schedule.
 * n_bins must be a multiple of n_groups; bad sizes or indices are
 * SA_ERR_INVALID_ARG. */
sa_status sa_lpt_schedule_grouped(const int64_t* loads, const int32_t* chunk_of_item, int32_t n_items,
                                  int32_t n_chunks, int32_t n_groups, int32_t n_bins,
                                  int32_t* bin_of_item, int32_t* bin_offsets, int32_t* items_by_bin,
                                  int64_t* bin_load);

/* Reorders the items of every bin ascending by item index, in place (host,
 * synchronous).  The bins keep the same items and loads, so the makespan of
 * the placement is unchanged; only the order in which a persistent workgroup
 * walks its bin changes.  With prefill items numbered (b, h, m) head-major,
 * every workgroup then moves through the heads in the same order, so at any
 * moment the workgroups read the key and value blocks of the same few KV heads
 * and those blocks are served from the caches.  The S-HPLB pages fix only
 * which device (here: bin) an item goes to, not the order inside it.
 *   bin_offsets[n_bins+1]  [host] as written by sa_lpt_schedule
 *   items_by_bin[...]      [host] in/out
 * Invalid offsets are SA_ERR_INVALID_ARG. */
sa_status sa_lpt_order_bins(const int32_t* bin_offsets, int32_t n_bins, int32_t* items_by_bin);

/* Order of the items for the prefill work queue (host, synchronous): the
 * greedy longest-processing-time rule of the S-HPLB pages (§2.B, §2.2) applied
 * online by workgroups that each take the next item when they finish one,
 * with the items grouped by group_of_item: groups in ascending order, inside
 * a group the largest load first, equal loads in item order.  With the group
 * of a prefill tile set to its (sequence, KV head), the tiles running at any
 * moment read the keys and values of one KV head, which stay in the caches,
 * and every group still ends with its smallest tiles.
 *   loads[n_items]          [host] int64 >= 0
 *   group_of_item[n_items]  [host] int32, may be NULL (one group)
 *   order[n_items]          [host] out: item indices in queue order
 * Negative loads are SA_ERR_INVALID_ARG. */
sa_status sa_lpt_queue_order(const int64_t* loads, const int32_t* group_of_item, int32_t n_items,
                             int32_t* order);

/* The work-queue order in load tiers (host, synchronous): items by tier
 * t(load) = floor(tiers_per_octave * log2(max(load, 1))) descending, then group
 * ascending, then load descending, then item index.  The tier is computed
 * exactly in integers (the bit length of max(load, 1)^tiers_per_octave, minus
 * one).  The longest items still open the queue, as the greedy rule needs for
 * its tail, while items of one group run together inside a tier.
 *   loads[n_items]          [host] int64 in [0, 2^15)
 *   group_of_item[n_items]  [host] int32, may be NULL (one group)
 *   tiers_per_octave        1, 2 or 4
 *   order[n_items]          [host] out: item indices in queue order
 * Loads outside [0, 2^15) or another tiers_per_octave are SA_ERR_INVALID_ARG. */
sa_status sa_lpt_queue_order_tiered(const int64_t* loads, const int32_t* group_of_item, int32_t n_items,
                                    int32_t tiers_per_octave, int32_t* order);

/* The work queue cut into partitions, one per cache domain (host,
 * synchronous).  MI355X has 8 XCDs, each with its own L2, and workgroup w of a
 * launch runs on XCD w mod 8; with one partition per XCD, the workgroups of an
 * XCD take the tiles placed on it, so the key and value blocks they gather are
 * shared through that XCD's L2.  The tiered order of sa_lpt_queue_order_tiered
 * is cut into units: runs of items of one (load tier, group), at most
 * chunk_items long (0: no limit).  Whole groups would keep the longest tiles of
 * a heavy group on one XCD, where they cannot all start at once; units of one
 * tier spread them over the XCDs while the workgroups of an XCD still work on
 * one group at a time.  The units go onto the partitions by the greedy longest-processing-time
 * rule of the S-HPLB pages (§2.B, §2.2) on their loads (least loaded partition
 * first, lower index on ties); inside a partition the items keep the tiered
 * order.  A workgroup whose partition is empty moves to the next ones in turn
 * (sa_sparse_attn_prefill_queues), so the tail is balanced across the chip.
 *   loads[n_items]               [host] int64 in [0, 2^15)
 *   group_of_item[n_items]       [host] int32 in [0, n_groups)
 *   n_queues                     1 .. 16
 *   tiers_per_octave             1, 2 or 4
 *   chunk_items                  items per unit at most, 0 = no limit
 *   order[n_items]               [host] out: items, partition after partition
 *   queue_offsets[n_queues + 1]  [host] out: partition i is order[off[i] .. off[i+1])
 * Out-of-range groups, loads or sizes are SA_ERR_INVALID_ARG. */
sa_status sa_lpt_queue_partition(const int64_t* loads, const int32_t* group_of_item, int32_t n_items,
                                 int32_t n_groups, int32_t n_queues, int32_t tiers_per_octave,
                                 int32_t chunk_items, int32_t* order, int32_t* queue_offsets);

/* Blocks kept per prefill row, from the budget rule alone (no data needed):
 * counts[b][h][m] for m < ceil(q_len/block_size) ([host] out, int32), and the
 * maximum over all rows in *kmax ([host] out, may be NULL).  These are the
 * item loads for sa_lpt_schedule (item = (b*n_q_heads + h)*n_blocks + m). */
sa_status sa_prefill_block_counts(const sa_attn_desc* desc, const sa_head_budget* budgets,
                                  int32_t* counts, int32_t* kmax);

/* Blocks kept per decode head (counts[h], [host] out) and their maximum. */
sa_status sa_decode_block_counts(const sa_attn_desc* desc, const sa_head_budget* budgets,
                                 int32_t* counts, int32_t* kmax);

/* ---------------------------------------------------------------- selection */

/* Bytes of fp32 pooled keys the decode selection reads: one array
 * [batch][n_kv_heads][ceil(kv_len/g)][head_dim] per distinct granularity g of
 * the heads that score (heads whose budget exceeds their forced blocks),
 * concatenated in ascending g. */
size_t sa_decode_pooled_size(const sa_attn_desc* desc, const sa_head_budget* budgets);

/* Build the decode pooled-key cache described above from k [dev] into
 * k_pooled [dev] (mean of each block's key rows in fp32; a short last block is
 * averaged over the rows it has). */
sa_status sa_pool_keys_decode(const sa_attn_desc* desc, const sa_head_budget* budgets,
                              const void* k, float* k_pooled, void* stream);

size_t sa_select_workspace_size(const sa_attn_desc* desc, const sa_head_budget* budgets,
                                int32_t kmax);

/* Top-k block selection.
 * prefill (q_len == kv_len): pools Q and K into fp32 block means (workspace),
 *   scores s[h][m][n] = scale * <Qbar[h][m], Kbar[h/G][n]> for n <= m, selects.
 *   k_pooled must be NULL.
 * decode (q_len == 1): scores s[h][n] = scale * <q[h], Kbar_g[h/G][n]> against
 *   the pooled-key cache k_pooled [dev] from sa_pool_keys_decode (NULL: pool
 *   from k into the workspace first).
 * Outputs [dev]: block_idx int32, prefill [batch][n_q_heads][n_blocks][kmax],
 * decode [batch][n_q_heads][kmax]: the kept blocks in ascending order, -1
 * padded; block_cnt int32 [batch][n_q_heads][n_blocks] (prefill) or
 * [batch][n_q_heads] (decode).  kmax must be >= the largest count
 * (sa_*_block_counts).
 * key_norms [dev] fp32 [batch][n_kv_heads][n_blocks], prefill only (NULL:
 * not written; must be NULL for decode): the largest Euclidean norm of a key
 * row of each key block, computed in fp32 from the same pass over k that
 * pools it.  sa_sparse_attn_prefill* take it to skip work (see there). */
sa_status sa_select_blocks(const sa_attn_desc* desc, const sa_head_budget* budgets,
                           const void* q, const void* k, const float* k_pooled,
                           int32_t* block_idx, int32_t* block_cnt, int32_t kmax,
                           float* key_norms, void* workspace, size_t workspace_bytes, void* stream);

/* The whole host schedule of a prefill layer's attention tiles in one call
 * (host, synchronous): block counts from the budgets (the tile loads), the
 * group keys, and the placement, using the calls above.  Tile item =
 * (b * n_q_heads + h) * n_blocks + m, n_tiles = batch * n_q_heads * n_blocks.
 *   kind SA_SCHED_GRID: one workgroup per tile in natural order; nothing is
 *        written (*n_offsets = 0).
 *   kind SA_SCHED_BINS: sa_lpt_schedule of the loads onto n_bins bins.
 *   kind SA_SCHED_BINS_XCD: sa_lpt_schedule_grouped: chunks of xcd_chunk
 *        query blocks of one (sequence, KV head) onto xcd_groups cache
 *        partitions, then the greedy rule inside each (n_bins a multiple of
 *        xcd_groups).
 *   Bins (both kinds) are walked in ascending item order (bin_order 0,
 *   sa_lpt_order_bins) or in assignment order (1).
 *   kind SA_SCHED_QUEUE: one order for the work queue, by queue_group:
 *     SA_QUEUE_KV_TIERS  load tiers of a quarter octave, heaviest first,
 *                        grouped by (sequence, KV head) inside a tier; with
 *                        n_queues > 1 cut into that many partitions
 *                        (sa_lpt_queue_partition, runs of at most queue_chunk
 *                        tiles, 0 = no limit);
 *     SA_QUEUE_KV        grouped by (sequence, KV head), longest first inside;
 *     SA_QUEUE_HEAD      grouped by (sequence, query head), the head with the
 *                        largest total load first (lower index on ties),
 *                        longest first inside;
 *     SA_QUEUE_FLAT      longest first;
 *     SA_QUEUE_AUTO      SA_QUEUE_FLAT on one queue for up to 256 query blocks
 *                        per head (a tile is then a large share of a
 *                        workgroup's work and the start of the longest tiles
 *                        decides the tail), else SA_QUEUE_KV_TIERS in n_queues
 *                        partitions (the workgroups of an XCD share a KV
 *                        head's blocks in its L2); *n_offsets tells which.
 *   items    [host] int32 [n_tiles] out (kinds other than GRID)
 *   offsets  [host] int32 out: bins: [n_bins + 1] bin offsets; queue:
 *            [n_queues + 1] partition offsets (n_queues 1 unless KV_TIERS)
 *   n_offsets [host] out: entries written to offsets
 *   bin_load [host] int64 [n_bins] out, bins only (may be NULL)
 * Sizes outside their ranges are SA_ERR_INVALID_ARG. */
enum { SA_SCHED_GRID = 0, SA_SCHED_BINS = 1, SA_SCHED_BINS_XCD = 2, SA_SCHED_QUEUE = 3 };
enum { SA_QUEUE_KV_TIERS = 0, SA_QUEUE_KV = 1, SA_QUEUE_HEAD = 2, SA_QUEUE_FLAT = 3, SA_QUEUE_AUTO = 4 };
typedef struct {
  int32_t kind;
  int32_t n_bins;       /* bins: number of bins (>= 1) */
  int32_t bin_order;    /* bins: 0 item order, 1 assignment order */
  int32_t xcd_groups;   /* SA_SCHED_BINS_XCD: cache partitions */
  int32_t xcd_chunk;    /* SA_SCHED_BINS_XCD: query blocks per chunk */
  int32_t queue_group;  /* SA_SCHED_QUEUE: SA_QUEUE_* */
  int32_t n_queues;     /* SA_SCHED_QUEUE with SA_QUEUE_KV_TIERS or SA_QUEUE_AUTO: 1 .. 16 */
  int32_t queue_chunk;  /* SA_SCHED_QUEUE with SA_QUEUE_KV_TIERS: run length limit */
} sa_prefill_schedule_opts;

sa_status sa_prefill_schedule(const sa_attn_desc* desc, const sa_head_budget* budgets,
                              const sa_prefill_schedule_opts* opts, int32_t* items, int32_t* offsets,
                              int32_t* n_offsets, int64_t* bin_load);

/* ---------------------------------------------------------------- attention */

size_t sa_prefill_workspace_size(const sa_attn_desc* desc, int32_t kmax, int32_t n_bins);

/* Causal block-sparse prefill attention.  Row t of query block m of head h
 * attends to keys t' <= t of the blocks block_idx[b][h][m][0..block_cnt-1] of
 * KV head h/G: o = softmax(scale * q k^T) v over those keys.
 *   q, k, v [dev] dtype desc->dtype; o [dev] fp32 if out_f32 else desc->dtype;
 *   lse [dev] fp32 [batch][n_q_heads][q_len] natural-log sum-exp (may be NULL).
 *   Schedule over the tiles item = (b*n_q_heads + h)*n_blocks + m, one of:
 *   - bins: bin_offsets [dev] (n_bins+1) and items_by_bin [dev] from
 *     sa_lpt_schedule; one persistent workgroup walks each bin;
 *   - work queue: bin_offsets NULL, items_by_bin [dev] one global order of all
 *     tiles (longest first is the greedy longest-processing-time rule run
 *     online); n_bins persistent workgroups each take the next tile of the
 *     order when they finish one.  The counter lives in workspace (>= 4 bytes,
 *     sa_prefill_workspace_size) and is reset by the call on the stream, so
 *     calls that share a workspace must not overlap;
 *   - both NULL: one workgroup per tile in natural order (n_bins ignored).
 *   Every tile must appear exactly once.  workspace may be NULL except in the
 *   work-queue mode.
 *   key_norms [dev] fp32 [batch][n_kv_heads][n_blocks] (may be NULL): for each
 *   key block an upper bound of the Euclidean norm of its key rows, as
 *   sa_select_blocks writes it for the same k.  The kernel keeps the softmax
 *   in the exp2 domain relative to a running max per row, which it must raise
 *   before a score could push a probability past what fp32 can accumulate.
 *   With the table, a step whose scores are bounded by scale * |q| * (the
 *   block's bound) <= running max + 64 (in log2 units) needs no row max (the
 *   first step of a tile always takes it); without it, every step takes the
 *   row max.  The normalised result is the same softmax either way (the
 *   running max cancels; only the bf16 rounding of the probabilities moves).
 *   A table that is not an upper bound for k can overflow the accumulators;
 *   with sa_set_debug_checks on, the host recomputes the bound from k and
 *   rejects such a table (SA_ERR_INVALID_ARG) before the launch. */
sa_status sa_sparse_attn_prefill(const sa_attn_desc* desc, const void* q, const void* k,
                                 const void* v, void* o, float* lse, const int32_t* block_idx,
                                 const int32_t* block_cnt, int32_t kmax, const float* key_norms,
                                 const int32_t* bin_offsets, const int32_t* items_by_bin,
                                 int32_t n_bins, int32_t out_f32, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* sa_sparse_attn_prefill on a work queue cut into n_queues partitions (from
 * sa_lpt_queue_partition): n_workgroups persistent workgroups, workgroup w
 * starting on partition w mod n_queues and moving on to the following
 * partitions once its own is empty; every workgroup has tried every partition
 * before it ends.  n_queues = 1 is the single queue of sa_sparse_attn_prefill.
 *   queue_offsets[n_queues + 1]  [host] 0 = off[0] <= ... <= off[n_queues] = tiles
 *   order[tiles]                 [dev] every tile exactly once
 *   workspace                    [dev] >= 4 * n_queues bytes (the counters), reset
 *                                by the call on the stream; calls sharing it must
 *                                not overlap
 * Bad offsets, n_queues outside [1, 16] or n_workgroups < 1 are
 * SA_ERR_INVALID_ARG; otherwise as sa_sparse_attn_prefill. */
sa_status sa_sparse_attn_prefill_queues(const sa_attn_desc* desc, const void* q, const void* k,
                                        const void* v, void* o, float* lse, const int32_t* block_idx,
                                        const int32_t* block_cnt, int32_t kmax, const float* key_norms,
                                        const int32_t* queue_offsets, int32_t n_queues,
                                        const int32_t* order, int32_t n_workgroups, int32_t out_f32,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* A prefill launch that records when each workgroup ran, to measure how well a
 * schedule fills the chip to the end (the idle tail that head load balancing
 * removes: "S-HPLB: Efficient LLM Attention Serving via Sparsity-Aware Head
 * Parallelism Load Balance", Italian summary §1 and §4).  Arguments as
 * sa_sparse_attn_prefill (queue_offsets NULL: bins, single queue or natural
 * order) or as sa_sparse_attn_prefill_queues (queue_offsets and n_queues set,
 * items_by_bin the order, n_bins the workgroup count).
 *   wg_times [dev] uint64 [2 * grid], 8-byte aligned, grid = n_bins (bins,
 *   queues) or the tile count (natural order): workgroup w writes the GPU's
 *   constant clock (s_memrealtime) when it starts to wg_times[2 w] and when it
 *   finishes to wg_times[2 w + 1].  The clock's rate is the device's wall-clock
 *   rate (hipDeviceAttributeWallClockRate). */
sa_status sa_sparse_attn_prefill_timed(const sa_attn_desc* desc, const void* q, const void* k,
                                       const void* v, void* o, float* lse, const int32_t* block_idx,
                                       const int32_t* block_cnt, int32_t kmax, const float* key_norms,
                                       const int32_t* bin_offsets, const int32_t* items_by_bin,
                                       int32_t n_bins, const int32_t* queue_offsets, int32_t n_queues,
                                       int32_t out_f32, uint64_t* wg_times, void* workspace,
                                       size_t workspace_bytes, void* stream);

size_t sa_decode_workspace_size(const sa_attn_desc* desc, const sa_head_budget* budgets,
                                int32_t kmax);

/* Block-sparse decode attention: the query of head h attends to the tokens of
 * its selected blocks (granularity budgets[h].granularity) of KV head h/G.  The
 * KV tokens of a group are read once for all its query heads (union of their
 * selections, per-head masks).  q [dev] [batch][n_q_heads][head_dim]; k, v
 * [dev] cache; o [dev] like q (fp32 if out_f32); lse [dev] fp32
 * [batch][n_q_heads] (may be NULL). */
sa_status sa_sparse_attn_decode(const sa_attn_desc* desc, const sa_head_budget* budgets,
                                const void* q, const void* k, const void* v, void* o,
                                float* lse, const int32_t* block_idx, const int32_t* block_cnt,
                                int32_t kmax, int32_t out_f32, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Size of the fixed scratch array of sa_sparse_attn_decode_noalloc (one per
 * GPU, held until the process ends): 16 MiB.  The 128K-token, 16-sequence,
 * 32/8-head decode step needs 6.3 MiB (sa_decode_workspace_size). */
#define SA_DECODE_SCRATCH_BYTES (16u << 20)

/* sa_sparse_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It calls no allocating routine; its
 * scratch is a fixed array of SA_DECODE_SCRATCH_BYTES in device memory, one per
 * GPU (looked up on the first call on a device, with that device current).
 * Arguments, layouts and results are those of sa_sparse_attn_decode (same
 * kernels, bitwise the same output).  Returns SA_ERR_WORKSPACE, before any
 * launch, when sa_decode_workspace_size(desc, budgets, kmax) exceeds
 * SA_DECODE_SCRATCH_BYTES.  Every call on one GPU uses that GPU's one array:
 * calls that overlap on one GPU (several streams or threads at once) race and
 * must be serialised by the caller.  Nothing in the array needs to start at
 * zero; it keeps the last call's contents. */
sa_status sa_sparse_attn_decode_noalloc(const sa_attn_desc* desc, const sa_head_budget* budgets,
                                        const void* q, const void* k, const void* v, void* o,
                                        float* lse, const int32_t* block_idx,
                                        const int32_t* block_cnt, int32_t kmax, int32_t out_f32,
                                        void* stream);

/* ---------------------------------------------------------------- calibration */

/* Offline calibration of per-head budgets: each head gets the budget that keeps
 * a share of its attention weight, and budget is shifted from heads that need
 * little to heads that need much with the total fixed, maximising the lowest
 * head's share ("S-HPLB: Efficient LLM Attention Serving via Sparsity-Aware
 * Head Parallelism Load Balance", Italian summary §2.A, Chinese summary §2.1). */

/* Attention mass per block pair: mass[b][h][m][n] = sum over the query rows t
 * of block m of head h of their exact causal softmax probabilities
 * softmax(scale q_t k^T) on the keys of block n (n <= m), zero for n > m.
 * Row m sums to the number of query rows in block m.  Prefill descriptor
 * (q_len == kv_len), bf16, block_size 128.  q, k [dev]; mass [dev] fp32
 * [batch][n_q_heads][n_blocks][n_blocks], written completely.  Costs two
 * passes of dense causal Q K^T: meant for calibration inputs, not the path. */
sa_status sa_block_attention_mass(const sa_attn_desc* desc, const void* q, const void* k, float* mass,
                                  void* stream);

/* Recovery table (host, synchronous): recovery[h][i] = mean over (sequence b,
 * query block m) of the share of row mass[b][h][m][0..m] kept by the row's best
 * selection at ratio r = (i+1) * step_q16: the forced blocks (budgets[h].n_sink
 * first, n_local last) plus the heaviest others (ties to the lowest index), k
 * blocks in all by the budget rule with budgets[h].min_blocks.  Kept and total
 * mass are summed in ascending block order in double.  mass [host] fp32
 * [batch][n_heads][n_blocks][n_blocks] (from sa_block_attention_mass);
 * recovery [host] double [n_heads][65536 / step_q16]; step_q16 divides 65536.
 * The ratio and granularity fields of budgets are not used. */
sa_status sa_budget_recovery(const float* mass, int32_t batch, int32_t n_heads, int32_t n_blocks,
                             const sa_head_budget* budgets, int32_t step_q16, double* recovery);

/* Output deviation per query head, the output-aware budget criterion of
 * "Fluxion" (Italian summary, Intuizioni Chiave 1: a budget judged by how far
 * it moves the head's attention output, not by the attention weight it keeps):
 *   dev[h] = sqrt(sum (o_approx - o_ref)^2) / sqrt(sum o_ref^2)
 * over every sequence, query row and channel of head h, summed in double in a
 * fixed order (bitwise reproducible); 0 where o_ref is all zero.  o_approx is
 * typically sa_sparse_attn_prefill's fp32 output (out_f32) at a candidate
 * budget and o_ref the same at ratio 1 (every block).  Over a grid of ratios
 * this gives a quality table (1 - dev) for sa_budget_shift.
 *   o_approx, o_ref [dev] fp32 with desc's o layout (o_stride, q_len rows,
 *                   head_dim contiguous), 16-byte aligned; head_dim and the
 *                   strides multiples of 4
 *   dev             [dev] double [n_q_heads]
 * One workgroup per head: an offline calibration step, not the path. */
sa_status sa_output_deviation(const sa_attn_desc* desc, const float* o_approx, const float* o_ref,
                              double* dev, void* stream);

/* Max-min budget shifting (host, synchronous) on a recovery table: every head
 * starts at total_q16 / n_heads (a whole number of steps); while the head with
 * the lowest recovery (lowest index on ties) can grow and another head can give
 * one step and still stay strictly above it (the one that stays highest, lowest
 * index on ties), one step moves.  For tables that grow with the ratio this
 * reaches the largest possible lowest recovery.  ratio_q16 [host] [n_heads]:
 * the shifted ratios, summing to total_q16. */
sa_status sa_budget_shift(const double* recovery, int32_t n_heads, int32_t step_q16, int64_t total_q16,
                          uint32_t* ratio_q16);

/* ---------------------------------------------------------------- paged KV */

/* A decode KV cache held in pages of page_size tokens, each KV head with its
 * own pool of physical pages: the page-based KV substrate that partitions of
 * any granularity map onto, with physical pages per attention head ("Unifying
 * Sparse Attention with Hierarchical Memory for Scalable Long-Context LLM
 * Serving" (Spin), §2.A partition abstraction and §2.B per-head physical
 * pages).
 *   K (and V) pool of KV head j: pages_per_head * page_size rows of head_dim
 *   elements starting at k + j * desc->k_stride[1]; row r (token r % page_size
 *   of physical page r / page_size) at + r * desc->k_stride[2].
 *   desc->k_stride[0] / v_stride[0] are not used.
 *   table [dev] int32 [batch][n_kv_heads][max_pages]: physical page (index into
 *   that KV head's pool) of logical page p = token / page_size of sequence b.
 * page_size is a multiple of 64, so every selection block (16, 32 or 64 tokens)
 * lies in one page; max_pages >= ceil(kv_len / page_size); one pool spans
 * < 2 GiB.  Entries outside [0, pages_per_head) read as zero keys and values.
 * Rows of a page past the cache end must hold finite values (they get
 * probability zero).  Owned by the caller, read only. */
typedef struct {
  const int32_t* table;
  int32_t page_size;
  int32_t max_pages;
  int32_t pages_per_head;
} sa_kv_pages;

/* sa_pool_keys_decode over a paged K cache (bf16 or fp32): the same pooled-key
 * cache, bit for bit, as the contiguous cache holding the same tokens. */
sa_status sa_pool_keys_decode_paged(const sa_attn_desc* desc, const sa_head_budget* budgets,
                                    const void* k_pages, const sa_kv_pages* pages, float* k_pooled,
                                    void* stream);

/* sa_sparse_attn_decode over a paged bf16 cache: the same results, bit for bit,
 * as over the contiguous cache holding the same tokens (the same arithmetic in
 * the same order; only the row addresses differ).  Workspace as
 * sa_decode_workspace_size.  fp32 caches return SA_ERR_UNSUPPORTED. */
sa_status sa_sparse_attn_decode_paged(const sa_attn_desc* desc, const sa_head_budget* budgets,
                                      const void* q, const void* k_pages, const void* v_pages,
                                      const sa_kv_pages* pages, void* o, float* lse,
                                      const int32_t* block_idx, const int32_t* block_cnt, int32_t kmax,
                                      int32_t out_f32, void* workspace, size_t workspace_bytes,
                                      void* stream);


/* ------------------------------------------------------------ measurement */

/* The bf16 matrix-core rate the GPU sustains: the denominator that the
 * attention kernels' achieved rate is set beside, next to the published dense
 * bf16 peak (MI355X: 2.5 PFLOP/s at 2.4 GHz).  n_workgroups workgroups of four
 * waves; every wave runs 8 independent accumulation chains of iters
 * v_mfma_f32_32x32x16_bf16 each, so the work is exactly
 *   n_workgroups * 4 * 8 * iters * 32768 flops.
 * operands = 0: every operand is 1.0 and every accumulator element ends at
 *   16 * iters; sink entries are 128 * iters (exact).
 * operands = 1: pseudo-random bf16 operands in [-1, 1), as matrix work on real
 *   data has (the chip's power limit holds a lower clock for them).  Lane l of
 *   global thread t = 256 * workgroup + thread holds four A and four B
 *   fragments; element e (0..7) of fragment f (A: f = 0..3, B: f = 4..7) is
 *   bf16 of ((h & 0xffff) - 32768) / 32768, rounded to nearest-even, with
 *   h = lowbias32(64 t + 8 f + e) (x ^= x >> 16; x *= 0x7feb352d;
 *   x ^= x >> 15; x *= 0x846ca68b; x ^= x >> 16, on uint32).  Chain c
 *   multiplies A[c % 4] (rows: lane % 32, k: 8 * (lane / 32) + e) by B[c % 4]
 *   (columns: lane % 32, same k); sink[t] = sum over c of element c of chain
 *   c's accumulator, i.e. iters times the (row 8 (c / 4) + 4 (lane / 32) +
 *   c % 4, column lane % 32) entry of that chain's 32 x 32 product, summed in
 *   fp32.
 *   sink [dev] fp32 [n_workgroups * 256]: the proof the work ran; owned by the
 *        caller.
 * n_workgroups in [1, 1 << 20], iters in [1, 65536], operands in {0, 1};
 * asynchronous on stream. */
sa_status sa_measure_mfma_peak(int32_t n_workgroups, int32_t iters, int32_t operands, float* sink, void* stream);

/* The HBM streaming-read rate the GPU sustains: the denominator for the
 * decode path, which reads its selected KV blocks once (published MI355X
 * peak: 8 TB/s).  Grid-stride 16-byte non-temporal loads of the whole buffer,
 * n_workgroups workgroups of 256 threads.
 *   buf  [dev] bytes bytes, 16-byte aligned, bytes a multiple of 16; read only
 *   sink [dev] uint32 [n_workgroups * 256]: the XOR of all of them equals the
 *        XOR of every 32-bit word of buf (the proof every byte was read)
 * n_workgroups in [1, 1 << 20]; asynchronous on stream. */
sa_status sa_measure_hbm_read(const void* buf, int64_t bytes, int32_t n_workgroups, uint32_t* sink,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
