// C ABI of libsparse_attn.so: argument validation, workspace layout, the
// greedy longest-load-first scheduler (host) and kernel launches.
//
// Every entry point validates all of its arguments before the first launch;
// on error it returns a negative sa_status and records a message readable with
// sa_last_error() on the same thread.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <queue>
#include <string>
#include <utility>
#include <vector>

#include "../../include/sparse_attn.h"
#include "sa_device.hpp"
#include "sa_kernels.hpp"

namespace {

thread_local std::string g_err;

sa_status fail(sa_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

sa_status ok() {
  g_err.clear();
  return SA_OK;
}

sa_status hip_fail(hipError_t e, const char* what) {
  return fail(SA_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

sa_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n == 0) return fail(SA_ERR_NO_DEVICE, "no HIP device visible");
    return hip_fail(e, "hipGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_NO_DEVICE, "device index %d out of range", dev);
  int s = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(s, std::memory_order_relaxed);
    if (s == 2) return fail(SA_ERR_ARCH, "device %d is %s, the kernels are built for gfx950", dev, prop.gcnArchName);
  }
  if (s == 2) return fail(SA_ERR_ARCH, "device %d is not gfx950", dev);
  return SA_OK;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int elem_size(int dtype) { return dtype == SA_BF16 ? 2 : 4; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_prefill(const sa_attn_desc* d) { return d->q_len != 1 || d->kv_len == 1; }

sa_status check_desc(const sa_attn_desc* d, bool prefill) {
  if (!d) return fail(SA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(SA_ERR_INVALID_ARG, "batch/heads must be >= 1 (got %d, %d, %d)", d->batch, d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads % d->n_kv_heads)
    return fail(SA_ERR_INVALID_ARG, "n_q_heads %d not a multiple of n_kv_heads %d", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads > SA_MAX_HEADS) return fail(SA_ERR_UNSUPPORTED, "n_q_heads > %d", SA_MAX_HEADS);
  if (d->head_dim != 64 && d->head_dim != 128) return fail(SA_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", d->head_dim);
  if (d->dtype != SA_BF16 && d->dtype != SA_F32) return fail(SA_ERR_INVALID_ARG, "dtype %d", d->dtype);
  if (d->kv_len < 1) return fail(SA_ERR_INVALID_ARG, "kv_len %d", d->kv_len);
  if (!(d->softmax_scale >= 0.f) || std::isinf(d->softmax_scale))
    return fail(SA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (d->kernel_variant != 0 && d->kernel_variant != 1)
    return fail(SA_ERR_INVALID_ARG, "kernel_variant %d (0 or 1)", d->kernel_variant);
  if (prefill) {
    if (d->q_len != d->kv_len) return fail(SA_ERR_INVALID_ARG, "prefill needs q_len == kv_len");
    if (d->block_size != 64 && d->block_size != 128)
      return fail(SA_ERR_UNSUPPORTED, "block_size %d (64 or 128)", d->block_size);
    if (d->dtype == SA_F32 && d->block_size != 64) return fail(SA_ERR_UNSUPPORTED, "fp32 prefill needs block_size 64");
    if (cdiv(d->q_len, d->block_size) > 8192) return fail(SA_ERR_UNSUPPORTED, "more than 8192 blocks per row");
  } else {
    if (d->q_len != 1) return fail(SA_ERR_INVALID_ARG, "decode needs q_len == 1");
    if (d->kv_len > (1 << 24) * 16) return fail(SA_ERR_UNSUPPORTED, "kv_len too large");
  }
  const int es = elem_size(d->dtype);
  const int64_t* st[4] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
  for (int t = 0; t < 4; ++t) {
    for (int i = 0; i < 3; ++i) {
      if (st[t][i] < 0) return fail(SA_ERR_INVALID_ARG, "negative stride");
      if (!prefill && (t == 0 || t == 3) && i == 2) continue;
      if ((st[t][i] * es) % 16) return fail(SA_ERR_INVALID_ARG, "strides must be multiples of 16 bytes");
    }
    if (prefill || t == 1 || t == 2)
      if (st[t][2] < d->head_dim) return fail(SA_ERR_INVALID_ARG, "token stride < head_dim");
  }
  return SA_OK;
}

sa_status check_budgets(const sa_attn_desc* d, const sa_head_budget* b, bool prefill) {
  if (!b) return fail(SA_ERR_INVALID_ARG, "budgets is NULL");
  for (int h = 0; h < d->n_q_heads; ++h) {
    const sa_head_budget& x = b[h];
    if (x.min_blocks < 1) return fail(SA_ERR_INVALID_ARG, "head %d: min_blocks must be >= 1", h);
    if (x.n_sink < 0 || x.n_local < 0 || x.n_sink > 32767 || x.n_local > 32767)
      return fail(SA_ERR_INVALID_ARG, "head %d: bad n_sink/n_local", h);
    if (x.n_sink + x.n_local > x.min_blocks)
      return fail(SA_ERR_INVALID_ARG, "head %d: n_sink + n_local (%d) exceeds min_blocks %d", h, x.n_sink + x.n_local,
                  x.min_blocks);
    if (x.ratio_q16 > 65536u) return fail(SA_ERR_INVALID_ARG, "head %d: ratio_q16 > 65536", h);
    if (!prefill) {
      const int g = x.granularity;
      if (g != 16 && g != 32 && g != 64 && g != 128)
        return fail(SA_ERR_UNSUPPORTED, "head %d: granularity %d (16, 32, 64 or 128)", h, g);
    }
  }
  return SA_OK;
}

sa::HeadTable make_table(const sa_attn_desc* d, const sa_head_budget* b, bool prefill) {
  sa::HeadTable t;
  std::memset(&t, 0, sizeof t);
  for (int h = 0; h < d->n_q_heads; ++h) {
    t.min_blocks[h] = b[h].min_blocks;
    t.ratio_q16[h] = b[h].ratio_q16;
    t.n_sink[h] = int16_t(b[h].n_sink);
    t.n_local[h] = int16_t(b[h].n_local);
    t.gran[h] = int16_t(prefill ? d->block_size : b[h].granularity);
  }
  return t;
}

int forced_count(int n, int ns, int nl) {
  ns = std::min(ns, n);
  const int lo = std::max(ns, n - nl);
  return ns + (n - lo);
}

int decode_count(const sa_attn_desc* d, const sa_head_budget& b) {
  const int nc = int(cdiv(d->kv_len, b.granularity));
  return sa::budget_blocks(nc, b.min_blocks, b.ratio_q16);
}

bool decode_scores_head(const sa_attn_desc* d, const sa_head_budget& b) {
  const int nc = int(cdiv(d->kv_len, b.granularity));
  const int k = sa::budget_blocks(nc, b.min_blocks, b.ratio_q16);
  return k > forced_count(nc, b.n_sink, b.n_local) && k < nc;
}

// distinct granularities of the scoring heads, ascending
std::vector<int> decode_pools(const sa_attn_desc* d, const sa_head_budget* b) {
  std::vector<int> g;
  for (int h = 0; h < d->n_q_heads; ++h)
    if (decode_scores_head(d, b[h])) g.push_back(b[h].granularity);
  std::sort(g.begin(), g.end());
  g.erase(std::unique(g.begin(), g.end()), g.end());
  return g;
}

size_t pooled_elems(const sa_attn_desc* d, int g) {
  return size_t(d->batch) * d->n_kv_heads * cdiv(d->kv_len, g) * d->head_dim;
}

// ---- workspace layouts
// prefill: the pooled keys only (query pooling, scores and top-k share one kernel)
struct PrefillSelectWs {
  size_t kpool, total;
};
PrefillSelectWs prefill_select_ws(const sa_attn_desc* d) {
  const size_t nb = cdiv(d->q_len, d->block_size);
  PrefillSelectWs w;
  w.kpool = 0;
  w.total = align256(size_t(d->batch) * d->n_kv_heads * nb * d->head_dim * 4);
  return w;
}

struct DecodeSelectWs {
  size_t pooled, scores, total;
  int nc_max;
};
DecodeSelectWs decode_select_ws(const sa_attn_desc* d, const sa_head_budget* b, bool need_pool) {
  DecodeSelectWs w;
  w.nc_max = 1;
  for (int h = 0; h < d->n_q_heads; ++h)
    if (decode_scores_head(d, b[h])) w.nc_max = std::max<int>(w.nc_max, int(cdiv(d->kv_len, b[h].granularity)));
  w.pooled = 0;
  size_t pooled = 0;
  if (need_pool)
    for (int g : decode_pools(d, b)) pooled += pooled_elems(d, g) * 4;
  w.scores = align256(pooled);
  w.total = w.scores + align256(size_t(d->batch) * d->n_q_heads * w.nc_max * 4);
  return w;
}

constexpr int kChunkAtoms = 40;  // atoms per decode attention wave: about one full round of waves at 128K
constexpr int kAtomPad = 16;  // tokens an atom may reach past the cache end
constexpr int kMaxQueues = sa::PrefillParams::kMaxQueues;
// SA_QUEUE_AUTO: the largest query-block count per head that gets one queue, longest first
constexpr int32_t kAutoFlatBlocks = 256;  // work-queue partitions (one per XCD on MI355X)

struct DecodeAttnWs {
  size_t atoms, n_union, part_o, part_ml, total;
  int max_union, n_chunks;
};
DecodeAttnWs decode_attn_ws(const sa_attn_desc* d, const sa_head_budget* b) {
  const int G = d->n_q_heads / d->n_kv_heads;
  const int64_t n_atoms = cdiv(d->kv_len, sa::kAtom);
  int64_t mu = 1;
  for (int j = 0; j < d->n_kv_heads; ++j) {
    int64_t s = 0;
    for (int gi = 0; gi < G; ++gi) {
      const sa_head_budget& x = b[j * G + gi];
      s += int64_t(decode_count(d, x)) * (x.granularity / sa::kAtom);
    }
    mu = std::max(mu, std::min(s, n_atoms));
  }
  DecodeAttnWs w;
  w.max_union = int(mu);
  w.n_chunks = int(cdiv(mu, kChunkAtoms));
  const size_t bk = size_t(d->batch) * d->n_kv_heads;
  w.atoms = 0;
  w.n_union = align256(bk * w.max_union * 4);
  w.part_o = w.n_union + align256(bk * 4);
  w.part_ml = w.part_o + align256(bk * w.n_chunks * G * d->head_dim * 4);
  w.total = w.part_ml + align256(bk * w.n_chunks * G * sa::kPartMl * 4);
  return w;
}

float scale_of(const sa_attn_desc* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt(float(d->head_dim));
}

// ---------------------------------------------------------------- debug checks
// With checks on (SA_DEBUG_CHECKS set to anything but "0" in the environment
// when the library loads, or sa_set_debug_checks(1)), every attention call
// first copies the index tables its kernels read back to the host (which
// synchronises the stream) and rejects the call with SA_ERR_INVALID_ARG if one
// is out of range.  The kernels themselves skip entries they cannot use, so
// without the checks a corrupt table gives wrong attention but no fault.
std::atomic<int> g_debug{[] {
  const char* e = std::getenv("SA_DEBUG_CHECKS");
  return (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
}()};

// Whether the checks run for a call on stream st: they are on and st is not
// being captured into a graph (a capture does not allow the synchronisation
// and copies the checks need, and trying them would invalidate the caller's
// capture; the calls made before a capture, such as its warm-up, are checked).
bool debug_checks(hipStream_t st) {
  if (!g_debug.load()) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;  // the checks report their own error
  return cs == hipStreamCaptureStatusNone;
}

template <typename T>
sa_status fetch(std::vector<T>& host, const T* dev, size_t n, hipStream_t st) {
  host.resize(n);
  if (n == 0) return ok();
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess) e = hipMemcpy(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost);
  return e == hipSuccess ? ok() : hip_fail(e, "debug check copy");
}

// rows of ascending block lists: row r holds cnt[r] <= kmax entries, each in
// [0, limit(r)), strictly increasing (a repeated block would be attended twice)
template <typename Limit>
sa_status check_lists(const int32_t* block_idx, const int32_t* block_cnt, int64_t rows, int32_t kmax, Limit limit,
                      hipStream_t st, const char* what) {
  std::vector<int32_t> cnt, idx;
  sa_status s = fetch(cnt, block_cnt, size_t(rows), st);
  if (s || (s = fetch(idx, block_idx, size_t(rows) * size_t(kmax), st))) return s;
  for (int64_t r = 0; r < rows; ++r) {
    const int32_t c = cnt[r];
    if (c < 0 || c > kmax) return fail(SA_ERR_INVALID_ARG, "%s: block_cnt[%lld] = %d outside [0, %d]", what, (long long)r, c, kmax);
    const int32_t lim = limit(r);
    for (int32_t j = 0; j < c; ++j) {
      const int32_t n = idx[size_t(r) * kmax + j];
      if (n < 0 || n >= lim)
        return fail(SA_ERR_INVALID_ARG, "%s: block_idx[%lld][%d] = %d outside [0, %d)", what, (long long)r, j, n, lim);
      if (j > 0 && n <= idx[size_t(r) * kmax + j - 1])
        return fail(SA_ERR_INVALID_ARG, "%s: block_idx[%lld] not strictly increasing at %d", what, (long long)r, j);
    }
  }
  return ok();
}

// items: a permutation of [0, n); offsets (device, n_bins + 1): 0 .. n, non-decreasing
// the key-norm table of a prefill launch bounds every key row: for each
// (sequence, KV head, key block), the largest Euclidean norm of the block's
// rows, recomputed from k on the host, is at most the table entry (relative
// slack 1e-5 for the fp32 rounding of the two sums)
sa_status check_key_norms(const sa_attn_desc* d, const void* k, const float* key_norms, hipStream_t st) {
  const int64_t nb = cdiv(d->kv_len, d->block_size);
  const int es = elem_size(d->dtype), D = d->head_dim;
  std::vector<float> tab;
  sa_status s = fetch(tab, key_norms, size_t(d->batch) * d->n_kv_heads * nb, st);
  if (s) return s;
  std::vector<char> rows(size_t(d->kv_len) * D * es);
  for (int b = 0; b < d->batch; ++b)
    for (int h = 0; h < d->n_kv_heads; ++h) {
      const char* src = static_cast<const char*>(k) + (b * d->k_stride[0] + h * d->k_stride[1]) * int64_t(es);
      const hipError_t e = hipMemcpy2D(rows.data(), size_t(D) * es, src, size_t(d->k_stride[2]) * es, size_t(D) * es,
                                       size_t(d->kv_len), hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "debug check copy");
      for (int64_t n = 0; n < nb; ++n) {
        double m2 = 0.0;
        const int64_t t1 = std::min<int64_t>(d->kv_len, (n + 1) * d->block_size);
        for (int64_t t = n * d->block_size; t < t1; ++t) {
          double q2 = 0.0;
          for (int j = 0; j < D; ++j) {
            float x;
            if (es == 2) {
              uint16_t u;
              std::memcpy(&u, rows.data() + (size_t(t) * D + j) * 2, 2);
              const uint32_t w = uint32_t(u) << 16;
              std::memcpy(&x, &w, 4);
            } else {
              std::memcpy(&x, rows.data() + (size_t(t) * D + j) * 4, 4);
            }
            q2 += double(x) * x;
          }
          m2 = std::max(m2, q2);
        }
        const double want = std::sqrt(m2);
        const float got = tab[(size_t(b) * d->n_kv_heads + h) * nb + n];
        if (!(double(got) >= want * (1.0 - 1e-5)))
          return fail(SA_ERR_INVALID_ARG,
                      "prefill: key_norms[%d][%d][%lld] = %g below the largest key norm %g of the block", b, h,
                      (long long)n, double(got), want);
      }
    }
  return ok();
}

sa_status check_items(const int32_t* items, const int32_t* offsets, int32_t n_bins, int64_t n, hipStream_t st) {
  std::vector<int32_t> it, off;
  sa_status s = fetch(it, items, size_t(n), st);
  if (s) return s;
  std::vector<char> seen(size_t(n), 0);
  for (int64_t i = 0; i < n; ++i) {
    if (it[i] < 0 || it[i] >= n) return fail(SA_ERR_INVALID_ARG, "items_by_bin[%lld] = %d outside [0, %lld)", (long long)i, it[i], (long long)n);
    if (seen[it[i]]++) return fail(SA_ERR_INVALID_ARG, "tile %d listed twice in items_by_bin", it[i]);
  }
  if (!offsets) return ok();
  if ((s = fetch(off, offsets, size_t(n_bins) + 1, st))) return s;
  if (off[0] != 0 || off[n_bins] != n) return fail(SA_ERR_INVALID_ARG, "bin_offsets must run from 0 to %lld", (long long)n);
  for (int32_t b = 0; b < n_bins; ++b)
    if (off[b + 1] < off[b]) return fail(SA_ERR_INVALID_ARG, "bin_offsets decrease at bin %d", b);
  return ok();
}

// page-table entries of the logical pages that hold cache rows, in [0, pages_per_head)
sa_status check_table(const sa_attn_desc* d, const sa_kv_pages* pg, hipStream_t st) {
  std::vector<int32_t> t;
  const int64_t rows = int64_t(d->batch) * d->n_kv_heads;
  sa_status s = fetch(t, pg->table, size_t(rows) * size_t(pg->max_pages), st);
  if (s) return s;
  const int64_t used = cdiv(d->kv_len, pg->page_size);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t p = 0; p < used; ++p) {
      const int32_t e = t[size_t(r) * pg->max_pages + p];
      if (e < 0 || e >= pg->pages_per_head)
        return fail(SA_ERR_INVALID_ARG, "page table [%lld][%lld] = %d outside [0, %d)", (long long)(r / d->n_kv_heads),
                    (long long)p, e, pg->pages_per_head);
    }
  return ok();
}

}  // namespace

extern "C" {

int32_t sa_version(void) { return 10000; }

int32_t sa_set_debug_checks(int32_t on) { return g_debug.exchange(on ? 1 : 0); }

const char* sa_last_error(void) { return g_err.c_str(); }

sa_status sa_lpt_schedule(const int64_t* loads, int32_t n_items, int32_t n_bins, int32_t* bin_of_item,
                          int32_t* bin_offsets, int32_t* items_by_bin, int64_t* bin_load) {
  if (n_items < 0) return fail(SA_ERR_INVALID_ARG, "n_items < 0");
  if (n_bins < 1) return fail(SA_ERR_INVALID_ARG, "n_bins must be >= 1");
  if (n_items > 0 && (!loads || !bin_of_item || !items_by_bin)) return fail(SA_ERR_INVALID_ARG, "NULL array");
  if (!bin_offsets) return fail(SA_ERR_INVALID_ARG, "bin_offsets is NULL");
  for (int32_t i = 0; i < n_items; ++i)
    if (loads[i] < 0) return fail(SA_ERR_INVALID_ARG, "load of item %d is negative", i);
  // items by load, largest first; equal loads keep ascending item order
  std::vector<int32_t> order(n_items);
  for (int32_t i = 0; i < n_items; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return loads[a] > loads[b]; });
  // least-loaded bin first; equal loads: lower bin index
  using Entry = std::pair<int64_t, int32_t>;
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap;
  for (int32_t b = 0; b < n_bins; ++b) heap.push({0, b});
  std::vector<int32_t> count(n_bins, 0);
  std::vector<int64_t> load(n_bins, 0);
  for (int32_t i : order) {
    Entry e = heap.top();
    heap.pop();
    bin_of_item[i] = e.second;
    count[e.second] += 1;
    load[e.second] = e.first + loads[i];
    heap.push({load[e.second], e.second});
  }
  bin_offsets[0] = 0;
  for (int32_t b = 0; b < n_bins; ++b) bin_offsets[b + 1] = bin_offsets[b] + count[b];
  std::vector<int32_t> fill(bin_offsets, bin_offsets + n_bins);
  for (int32_t i : order) items_by_bin[fill[bin_of_item[i]]++] = i;  // assignment order
  if (bin_load)
    for (int32_t b = 0; b < n_bins; ++b) bin_load[b] = load[b];
  return ok();
}

sa_status sa_lpt_schedule_grouped(const int64_t* loads, const int32_t* chunk_of_item, int32_t n_items,
                                  int32_t n_chunks, int32_t n_groups, int32_t n_bins, int32_t* bin_of_item,
                                  int32_t* bin_offsets, int32_t* items_by_bin, int64_t* bin_load) {
  if (n_items < 0 || n_chunks < 1 || n_groups < 1 || n_bins < 1) return fail(SA_ERR_INVALID_ARG, "bad sizes");
  if (n_bins % n_groups) return fail(SA_ERR_INVALID_ARG, "n_bins %d is not a multiple of n_groups %d", n_bins, n_groups);
  if (n_items > 0 && (!loads || !chunk_of_item || !bin_of_item || !items_by_bin))
    return fail(SA_ERR_INVALID_ARG, "NULL array");
  if (!bin_offsets) return fail(SA_ERR_INVALID_ARG, "bin_offsets is NULL");
  std::vector<int64_t> cload(n_chunks, 0);
  for (int32_t i = 0; i < n_items; ++i) {
    if (loads[i] < 0) return fail(SA_ERR_INVALID_ARG, "load of item %d is negative", i);
    if (chunk_of_item[i] < 0 || chunk_of_item[i] >= n_chunks)
      return fail(SA_ERR_INVALID_ARG, "chunk of item %d out of range", i);
    cload[chunk_of_item[i]] += loads[i];
  }
  // level 1: chunks onto groups; level 2: each group's items onto its bins
  std::vector<int32_t> group_of_chunk(n_chunks), off1(n_groups + 1), tmp1(n_chunks);
  sa_status st = sa_lpt_schedule(cload.data(), n_chunks, n_groups, group_of_chunk.data(), off1.data(), tmp1.data(),
                                 nullptr);
  if (st) return st;
  const int32_t per = n_bins / n_groups;
  std::vector<std::vector<int32_t>> bin_items(n_bins);
  std::vector<int64_t> load(n_bins, 0);
  std::vector<int32_t> members;
  std::vector<int64_t> mload;
  for (int32_t g = 0; g < n_groups; ++g) {
    members.clear();
    mload.clear();
    for (int32_t i = 0; i < n_items; ++i)
      if (group_of_chunk[chunk_of_item[i]] == g) {
        members.push_back(i);
        mload.push_back(loads[i]);
      }
    const int32_t m = int32_t(members.size());
    std::vector<int32_t> b_of(m), off(per + 1), its(m);
    std::vector<int64_t> bl(per);
    if ((st = sa_lpt_schedule(mload.data(), m, per, b_of.data(), off.data(), its.data(), bl.data()))) return st;
    for (int32_t lb = 0; lb < per; ++lb) {
      const int32_t gb = lb * n_groups + g;  // bin gb runs on group gb % n_groups
      for (int32_t t = off[lb]; t < off[lb + 1]; ++t) bin_items[gb].push_back(members[its[t]]);
      load[gb] = bl[lb];
    }
  }
  bin_offsets[0] = 0;
  for (int32_t b = 0; b < n_bins; ++b) {
    bin_offsets[b + 1] = bin_offsets[b] + int32_t(bin_items[b].size());
    for (size_t t = 0; t < bin_items[b].size(); ++t) {
      items_by_bin[bin_offsets[b] + t] = bin_items[b][t];
      bin_of_item[bin_items[b][t]] = b;
    }
    if (bin_load) bin_load[b] = load[b];
  }
  return ok();
}

sa_status sa_lpt_order_bins(const int32_t* bin_offsets, int32_t n_bins, int32_t* items_by_bin) {
  if (n_bins < 1 || !bin_offsets) return fail(SA_ERR_INVALID_ARG, "bin_offsets is NULL or n_bins < 1");
  if (bin_offsets[0] != 0) return fail(SA_ERR_INVALID_ARG, "bin_offsets[0] must be 0");
  for (int32_t b = 0; b < n_bins; ++b)
    if (bin_offsets[b + 1] < bin_offsets[b]) return fail(SA_ERR_INVALID_ARG, "bin_offsets must not decrease");
  if (bin_offsets[n_bins] > 0 && !items_by_bin) return fail(SA_ERR_INVALID_ARG, "items_by_bin is NULL");
  for (int32_t b = 0; b < n_bins; ++b) std::sort(items_by_bin + bin_offsets[b], items_by_bin + bin_offsets[b + 1]);
  return ok();
}

sa_status sa_lpt_queue_order(const int64_t* loads, const int32_t* group_of_item, int32_t n_items, int32_t* order) {
  if (n_items < 0) return fail(SA_ERR_INVALID_ARG, "n_items < 0");
  if (n_items > 0 && (!loads || !order)) return fail(SA_ERR_INVALID_ARG, "loads or order is NULL");
  for (int32_t i = 0; i < n_items; ++i) {
    if (loads[i] < 0) return fail(SA_ERR_INVALID_ARG, "negative load at item %d", i);
    order[i] = i;
  }
  const auto group = [&](int32_t i) { return group_of_item ? group_of_item[i] : 0; };
  std::stable_sort(order, order + n_items, [&](int32_t a, int32_t b) {
    if (group(a) != group(b)) return group(a) < group(b);
    return loads[a] > loads[b];
  });
  return ok();
}

sa_status sa_lpt_queue_order_tiered(const int64_t* loads, const int32_t* group_of_item, int32_t n_items,
                                    int32_t tiers_per_octave, int32_t* order) {
  if (n_items < 0) return fail(SA_ERR_INVALID_ARG, "n_items < 0");
  if (tiers_per_octave != 1 && tiers_per_octave != 2 && tiers_per_octave != 4)
    return fail(SA_ERR_INVALID_ARG, "tiers_per_octave %d (1, 2 or 4)", tiers_per_octave);
  if (n_items > 0 && (!loads || !order)) return fail(SA_ERR_INVALID_ARG, "loads or order is NULL");
  std::vector<int32_t> tier(n_items);
  for (int32_t i = 0; i < n_items; ++i) {
    if (loads[i] < 0 || loads[i] >= (1 << 15)) return fail(SA_ERR_INVALID_ARG, "load %lld at item %d outside [0, 2^15)",
                                                          (long long)loads[i], i);
    uint64_t p = 1;
    const uint64_t x = uint64_t(std::max<int64_t>(loads[i], 1));
    for (int32_t t = 0; t < tiers_per_octave; ++t) p *= x;  // < 2^60
    tier[i] = 63 - __builtin_clzll(p);                          // floor(log2(x^t))
    order[i] = i;
  }
  const auto group = [&](int32_t i) { return group_of_item ? group_of_item[i] : 0; };
  std::stable_sort(order, order + n_items, [&](int32_t a, int32_t b) {
    if (tier[a] != tier[b]) return tier[a] > tier[b];
    if (group(a) != group(b)) return group(a) < group(b);
    return loads[a] > loads[b];
  });
  return ok();
}

sa_status sa_lpt_queue_partition(const int64_t* loads, const int32_t* group_of_item, int32_t n_items,
                                 int32_t n_groups, int32_t n_queues, int32_t tiers_per_octave, int32_t chunk_items,
                                 int32_t* order, int32_t* queue_offsets) {
  if (n_items < 0 || n_groups < 1) return fail(SA_ERR_INVALID_ARG, "n_items < 0 or n_groups < 1");
  if (n_queues < 1 || n_queues > kMaxQueues)
    return fail(SA_ERR_INVALID_ARG, "n_queues %d outside [1, %d]", n_queues, kMaxQueues);
  if (chunk_items < 0) return fail(SA_ERR_INVALID_ARG, "chunk_items must be >= 0");
  if (chunk_items == 0) chunk_items = std::max<int32_t>(n_items, 1);  // no limit
  if (!queue_offsets || (n_items > 0 && (!loads || !group_of_item || !order)))
    return fail(SA_ERR_INVALID_ARG, "NULL array");
  for (int32_t i = 0; i < n_items; ++i)
    if (group_of_item[i] < 0 || group_of_item[i] >= n_groups)
      return fail(SA_ERR_INVALID_ARG, "group %d of item %d outside [0, %d)", group_of_item[i], i, n_groups);
  // the tiered order (validates the loads and tiers_per_octave)
  std::vector<int32_t> tiered(n_items);
  sa_status st = sa_lpt_queue_order_tiered(loads, group_of_item, n_items, tiers_per_octave, tiered.data());
  if (st) return st;
  const auto tier_of = [&](int32_t i) {
    uint64_t p = 1;
    const uint64_t x = uint64_t(std::max<int64_t>(loads[i], 1));
    for (int32_t t = 0; t < tiers_per_octave; ++t) p *= x;
    return 63 - __builtin_clzll(p);
  };
  // units: runs of the tiered order with one (tier, group), cut every chunk_items items
  std::vector<int32_t> unit_of_pos(n_items);
  std::vector<int64_t> uload;
  for (int32_t pos = 0, run = 0; pos < n_items; ++pos) {
    const int32_t i = tiered[pos];
    const bool same = pos > 0 && group_of_item[tiered[pos - 1]] == group_of_item[i] &&
                      tier_of(tiered[pos - 1]) == tier_of(i);
    run = same ? run + 1 : 0;
    if (!same || run % chunk_items == 0) uload.push_back(0);
    unit_of_pos[pos] = int32_t(uload.size()) - 1;
    uload.back() += loads[i];
  }
  // units onto queues by the greedy rule on their loads
  const int32_t n_units = int32_t(uload.size());
  std::vector<int32_t> queue_of_unit(n_units), uoff(n_queues + 1), uitems(n_units);
  if (n_units > 0 &&
      (st = sa_lpt_schedule(uload.data(), n_units, n_queues, queue_of_unit.data(), uoff.data(), uitems.data(), nullptr)))
    return st;
  // every queue keeps the tiered order of its items
  std::vector<int32_t> count(n_queues, 0);
  for (int32_t pos = 0; pos < n_items; ++pos) count[queue_of_unit[unit_of_pos[pos]]] += 1;
  queue_offsets[0] = 0;
  for (int32_t q = 0; q < n_queues; ++q) queue_offsets[q + 1] = queue_offsets[q] + count[q];
  std::vector<int32_t> fill(queue_offsets, queue_offsets + n_queues);
  for (int32_t pos = 0; pos < n_items; ++pos) order[fill[queue_of_unit[unit_of_pos[pos]]]++] = tiered[pos];
  return ok();
}

sa_status sa_prefill_block_counts(const sa_attn_desc* desc, const sa_head_budget* budgets, int32_t* counts,
                                  int32_t* kmax) {
  sa_status s = check_desc(desc, true);
  if (s) return s;
  if ((s = check_budgets(desc, budgets, true))) return s;
  const int nb = int(cdiv(desc->q_len, desc->block_size));
  int km = 0;
  for (int b = 0; b < desc->batch; ++b)
    for (int h = 0; h < desc->n_q_heads; ++h)
      for (int m = 0; m < nb; ++m) {
        const int k = sa::budget_blocks(m + 1, budgets[h].min_blocks, budgets[h].ratio_q16);
        if (counts) counts[((int64_t)b * desc->n_q_heads + h) * nb + m] = k;
        km = std::max(km, k);
      }
  if (kmax) *kmax = km;
  return ok();
}

sa_status sa_prefill_schedule(const sa_attn_desc* desc, const sa_head_budget* budgets,
                              const sa_prefill_schedule_opts* opts, int32_t* items, int32_t* offsets,
                              int32_t* n_offsets, int64_t* bin_load) {
  if (!opts || !n_offsets) return fail(SA_ERR_INVALID_ARG, "opts or n_offsets is NULL");
  sa_status st = check_desc(desc, true);
  if (st) return st;
  if ((st = check_budgets(desc, budgets, true))) return st;
  *n_offsets = 0;
  const sa_prefill_schedule_opts& o = *opts;
  if (o.kind == SA_SCHED_GRID) return ok();
  if (o.kind != SA_SCHED_BINS && o.kind != SA_SCHED_BINS_XCD && o.kind != SA_SCHED_QUEUE)
    return fail(SA_ERR_INVALID_ARG, "schedule kind %d", o.kind);
  const int32_t nb = int32_t(cdiv(desc->q_len, desc->block_size));
  const int32_t Hq = desc->n_q_heads, Hkv = desc->n_kv_heads, G = Hq / Hkv;
  const int64_t n64 = int64_t(desc->batch) * Hq * nb;
  if (n64 > INT32_MAX) return fail(SA_ERR_INVALID_ARG, "%lld tiles exceed int32", (long long)n64);
  const int32_t n = int32_t(n64);
  if (!items || !offsets) return fail(SA_ERR_INVALID_ARG, "items or offsets is NULL");
  std::vector<int32_t> cnt(n);
  if ((st = sa_prefill_block_counts(desc, budgets, cnt.data(), nullptr))) return st;
  std::vector<int64_t> loads(cnt.begin(), cnt.end());
  // item = (b * Hq + h) * nb + m
  const auto bh_of = [&](int32_t it) { return it / nb; };
  if (o.kind == SA_SCHED_QUEUE) {
    int32_t qgroup = o.queue_group, nq = o.n_queues;
    if (qgroup == SA_QUEUE_AUTO) {
      // Up to kAutoFlatBlocks query blocks per head, a tile is a large share of
      // a workgroup's work and the start of the longest tiles decides the
      // tail: plain longest first on one queue.  Beyond it, the tiered order
      // in per-XCD partitions, whose workgroups share a KV head's blocks in
      // their XCD's L2 (measured on MI355X: 32K tokens, 256 blocks, flat 3%
      // ahead; 64K and 128K, the partitions 4% ahead of any one queue).
      if (nb <= kAutoFlatBlocks) {
        qgroup = SA_QUEUE_FLAT;
        nq = 1;
      } else {
        qgroup = SA_QUEUE_KV_TIERS;
      }
    }
    std::vector<int32_t> group(n);
    switch (qgroup) {
      case SA_QUEUE_KV_TIERS:
      case SA_QUEUE_KV:
        for (int32_t it = 0; it < n; ++it) group[it] = bh_of(it) / G;  // (b, KV head) = (b * Hq + h) / G
        break;
      case SA_QUEUE_HEAD: {
        const int32_t n_bh = desc->batch * Hq;
        std::vector<int64_t> tot(n_bh, 0);
        for (int32_t it = 0; it < n; ++it) tot[bh_of(it)] += loads[it];
        std::vector<int32_t> by(n_bh), rank(n_bh);
        for (int32_t i = 0; i < n_bh; ++i) by[i] = i;
        std::stable_sort(by.begin(), by.end(), [&](int32_t a, int32_t b) { return tot[a] > tot[b]; });
        for (int32_t r = 0; r < n_bh; ++r) rank[by[r]] = r;
        for (int32_t it = 0; it < n; ++it) group[it] = rank[bh_of(it)];
        break;
      }
      case SA_QUEUE_FLAT:
        break;
      default:
        return fail(SA_ERR_INVALID_ARG, "queue_group %d", o.queue_group);
    }
    const int32_t* gp = qgroup == SA_QUEUE_FLAT ? nullptr : group.data();
    if (qgroup == SA_QUEUE_KV_TIERS && nq > 1) {
      if ((st = sa_lpt_queue_partition(loads.data(), gp, n, desc->batch * Hkv, nq, 4, o.queue_chunk, items,
                                       offsets)))
        return st;
      *n_offsets = nq + 1;
      return ok();
    }
    if (nq != 1 && nq != 0 && qgroup != SA_QUEUE_KV_TIERS)
      return fail(SA_ERR_INVALID_ARG, "n_queues > 1 needs queue_group SA_QUEUE_KV_TIERS");
    st = qgroup == SA_QUEUE_KV_TIERS ? sa_lpt_queue_order_tiered(loads.data(), gp, n, 4, items)
                                     : sa_lpt_queue_order(loads.data(), gp, n, items);
    if (st) return st;
    offsets[0] = 0;
    offsets[1] = n;
    *n_offsets = 2;
    return ok();
  }
  // static bins
  if (o.n_bins < 1) return fail(SA_ERR_INVALID_ARG, "n_bins must be >= 1");
  if (o.bin_order != 0 && o.bin_order != 1) return fail(SA_ERR_INVALID_ARG, "bin_order %d", o.bin_order);
  std::vector<int32_t> bin_of(n);
  if (o.kind == SA_SCHED_BINS_XCD) {
    if (o.xcd_groups < 1 || o.xcd_chunk < 1) return fail(SA_ERR_INVALID_ARG, "xcd_groups and xcd_chunk must be >= 1");
    // chunk = (b * Hkv + h / G) * n_m + m / xcd_chunk
    const int32_t n_m = int32_t(cdiv(nb, o.xcd_chunk));
    std::vector<int32_t> chunk(n);
    for (int32_t it = 0; it < n; ++it) {
      const int32_t bh = bh_of(it), m = it % nb;
      const int32_t b = bh / Hq, h = bh % Hq;
      chunk[it] = (b * Hkv + h / G) * n_m + m / o.xcd_chunk;
    }
    const int32_t n_chunks = desc->batch * Hkv * n_m;
    st = sa_lpt_schedule_grouped(loads.data(), chunk.data(), n, n_chunks, o.xcd_groups, o.n_bins, bin_of.data(),
                                 offsets, items, bin_load);
  } else {
    st = sa_lpt_schedule(loads.data(), n, o.n_bins, bin_of.data(), offsets, items, bin_load);
  }
  if (st) return st;
  if (o.bin_order == 0 && (st = sa_lpt_order_bins(offsets, o.n_bins, items))) return st;
  *n_offsets = o.n_bins + 1;
  return ok();
}

sa_status sa_decode_block_counts(const sa_attn_desc* desc, const sa_head_budget* budgets, int32_t* counts,
                                 int32_t* kmax) {
  sa_status s = check_desc(desc, false);
  if (s) return s;
  if ((s = check_budgets(desc, budgets, false))) return s;
  int km = 0;
  for (int h = 0; h < desc->n_q_heads; ++h) {
    const int k = decode_count(desc, budgets[h]);
    if (counts) counts[h] = k;
    km = std::max(km, k);
  }
  if (kmax) *kmax = km;
  return ok();
}

size_t sa_decode_pooled_size(const sa_attn_desc* desc, const sa_head_budget* budgets) {
  if (check_desc(desc, false) || check_budgets(desc, budgets, false)) return 0;
  size_t n = 0;
  for (int g : decode_pools(desc, budgets)) n += pooled_elems(desc, g) * 4;
  return n;
}

static sa::PageTable page_table_of(const sa_kv_pages* pages) {
  sa::PageTable t;
  t.table = pages ? pages->table : nullptr;
  t.page_size = pages ? pages->page_size : 0;
  t.max_pages = pages ? pages->max_pages : 0;
  t.pages_per_head = pages ? pages->pages_per_head : 0;
  return t;
}

static sa_status pool_decode_into(const sa_attn_desc* d, const sa_head_budget* b, const void* k, float* out,
                                  hipStream_t st, const sa_kv_pages* pages = nullptr) {
  size_t off = 0;
  for (int g : decode_pools(d, b)) {
    sa::PoolParams pp{};
    pp.x = k;
    pp.s0 = d->k_stride[0];
    pp.s1 = d->k_stride[1];
    pp.s2 = d->k_stride[2];
    pp.pages = page_table_of(pages);
    pp.out = out + off;
    pp.heads = d->n_kv_heads;
    pp.T = d->kv_len;
    pp.g = g;
    pp.nb = int(cdiv(d->kv_len, g));
    pp.blocks_per_wg = std::max(1, 256 / g);
    hipError_t e = sa::launch_pool(pp, d->dtype, d->head_dim, d->batch, st);
    if (e != hipSuccess) return hip_fail(e, "pool kernel launch");
    off += pooled_elems(d, g);
  }
  return SA_OK;
}

sa_status sa_pool_keys_decode(const sa_attn_desc* desc, const sa_head_budget* budgets, const void* k,
                              float* k_pooled, void* stream) {
  sa_status s = check_desc(desc, false);
  if (s) return s;
  if ((s = check_budgets(desc, budgets, false))) return s;
  if (!k || !k_pooled) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(k) || !aligned16(k_pooled)) return fail(SA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if ((s = check_device())) return s;
  if ((s = pool_decode_into(desc, budgets, k, k_pooled, (hipStream_t)stream))) return s;
  return ok();
}

// Checks of a paged cache description shared by the paged entry points.
static sa_status check_pages(const sa_attn_desc* d, const sa_kv_pages* pages) {
  if (!pages || !pages->table) return fail(SA_ERR_INVALID_ARG, "pages or pages->table is NULL");
  if (pages->page_size < 64 || pages->page_size % 64)
    return fail(SA_ERR_INVALID_ARG, "page_size %d is not a positive multiple of 64", pages->page_size);
  if (pages->pages_per_head < 1) return fail(SA_ERR_INVALID_ARG, "pages_per_head must be >= 1");
  if (int64_t(pages->max_pages) * pages->page_size < d->kv_len)
    return fail(SA_ERR_INVALID_ARG, "max_pages %d pages of %d tokens do not cover kv_len %d", pages->max_pages,
                pages->page_size, d->kv_len);
  if (reinterpret_cast<uintptr_t>(pages->table) & 3) return fail(SA_ERR_INVALID_ARG, "page table must be 4-byte aligned");
  const int64_t es = elem_size(d->dtype);
  const int64_t rows = int64_t(pages->pages_per_head) * pages->page_size;
  if ((rows + kAtomPad) * d->k_stride[2] * es >= (1ll << 31) || (rows + kAtomPad) * d->v_stride[2] * es >= (1ll << 31))
    return fail(SA_ERR_UNSUPPORTED, "one KV head's page pool must span < 2 GiB");
  return SA_OK;
}

sa_status sa_pool_keys_decode_paged(const sa_attn_desc* desc, const sa_head_budget* budgets, const void* k_pages,
                                    const sa_kv_pages* pages, float* k_pooled, void* stream) {
  sa_status s = check_desc(desc, false);
  if (s) return s;
  if ((s = check_budgets(desc, budgets, false))) return s;
  if ((s = check_pages(desc, pages))) return s;
  if (!k_pages || !k_pooled) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(k_pages) || !aligned16(k_pooled)) return fail(SA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if ((s = check_device())) return s;
  if ((s = pool_decode_into(desc, budgets, k_pages, k_pooled, (hipStream_t)stream, pages))) return s;
  return ok();
}

size_t sa_select_workspace_size(const sa_attn_desc* desc, const sa_head_budget* budgets, int32_t kmax) {
  (void)kmax;
  if (!desc) return 0;
  if (is_prefill(desc)) {
    if (check_desc(desc, true)) return 0;
    return prefill_select_ws(desc).total;
  }
  if (check_desc(desc, false) || check_budgets(desc, budgets, false)) return 0;
  return decode_select_ws(desc, budgets, true).total;
}

sa_status sa_select_blocks(const sa_attn_desc* desc, const sa_head_budget* budgets, const void* q, const void* k,
                           const float* k_pooled, int32_t* block_idx, int32_t* block_cnt, int32_t kmax,
                           float* key_norms, void* workspace, size_t workspace_bytes, void* stream) {
  if (!desc) return fail(SA_ERR_INVALID_ARG, "desc is NULL");
  const bool prefill = is_prefill(desc);
  sa_status s = check_desc(desc, prefill);
  if (s) return s;
  if ((s = check_budgets(desc, budgets, prefill))) return s;
  if (!q || !k || !block_idx || !block_cnt) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(q) || !aligned16(k) || (k_pooled && !aligned16(k_pooled)))
    return fail(SA_ERR_INVALID_ARG, "q, k and k_pooled must be 16-byte aligned");
  int32_t need = 0;
  if (reinterpret_cast<uintptr_t>(key_norms) & 3) return fail(SA_ERR_INVALID_ARG, "key_norms must be 4-byte aligned");
  if (!prefill && key_norms) return fail(SA_ERR_INVALID_ARG, "key_norms is for prefill only");
  if (prefill) {
    if (k_pooled) return fail(SA_ERR_INVALID_ARG, "k_pooled must be NULL for prefill");
    sa_prefill_block_counts(desc, budgets, nullptr, &need);
  } else {
    sa_decode_block_counts(desc, budgets, nullptr, &need);
  }
  if (kmax < need) return fail(SA_ERR_INVALID_ARG, "kmax %d < largest block count %d", kmax, need);
  if (prefill && cdiv(desc->q_len, desc->block_size) > sa::kSelMaxBlocks)
    return fail(SA_ERR_UNSUPPORTED, "%lld query blocks > %d", (long long)cdiv(desc->q_len, desc->block_size),
                sa::kSelMaxBlocks);
  const size_t ws_need = prefill ? prefill_select_ws(desc).total : decode_select_ws(desc, budgets, !k_pooled).total;
  if (!workspace || workspace_bytes < ws_need)
    return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws_need, workspace_bytes);
  if (!aligned16(workspace)) return fail(SA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if ((s = check_device())) return s;
  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  const float scale = scale_of(desc);
  const int D = desc->head_dim;
  const int G = desc->n_q_heads / desc->n_kv_heads;
  hipError_t e;
  sa::TopkParams tp{};
  std::memset(&tp, 0, sizeof tp);
  tp.idx = block_idx;
  tp.cnt = block_cnt;
  tp.kmax = kmax;
  tp.Hq = desc->n_q_heads;
  tp.heads = make_table(desc, budgets, prefill);
  if (prefill) {
    const PrefillSelectWs w = prefill_select_ws(desc);
    const int nb = int(cdiv(desc->q_len, desc->block_size));
    float* kp = reinterpret_cast<float*>(ws + w.kpool);
    sa::PoolParams pp{};
    pp.g = desc->block_size;
    pp.nb = nb;
    pp.T = desc->kv_len;
    pp.blocks_per_wg = 1;
    pp.x = k;
    pp.s0 = desc->k_stride[0];
    pp.s1 = desc->k_stride[1];
    pp.s2 = desc->k_stride[2];
    pp.out = kp;
    pp.heads = desc->n_kv_heads;
    pp.norm_max = key_norms;
    if ((e = sa::launch_pool(pp, desc->dtype, D, desc->batch, st)) != hipSuccess) return hip_fail(e, "pool K");
    sa::PrefillSelectParams sp{};
    sp.q = q;
    sp.qs0 = desc->q_stride[0];
    sp.qs1 = desc->q_stride[1];
    sp.qs2 = desc->q_stride[2];
    sp.kp = kp;
    sp.idx = block_idx;
    sp.cnt = block_cnt;
    sp.kmax = kmax;
    sp.Hq = desc->n_q_heads;
    sp.G = G;
    sp.S = desc->q_len;
    sp.NB = nb;
    sp.R = sa::sel_rows(nb);
    sp.rowlen = sa::sel_rowlen(nb);
    sp.n_mg = int(cdiv(nb, sp.R));
    sp.scale = scale;
    sp.heads = tp.heads;
    if ((e = sa::launch_select_prefill(sp, desc->dtype, D, desc->block_size, desc->batch, st)) != hipSuccess)
      return hip_fail(e, "prefill selection");
    return ok();
  }
  // decode
  const DecodeSelectWs w = decode_select_ws(desc, budgets, !k_pooled);
  const float* pooled = k_pooled;
  if (!pooled) {
    if ((s = pool_decode_into(desc, budgets, k, reinterpret_cast<float*>(ws + w.pooled), st))) return s;
    pooled = reinterpret_cast<const float*>(ws + w.pooled);
  }
  float* sc = reinterpret_cast<float*>(ws + w.scores);
  const std::vector<int> pools = decode_pools(desc, budgets);
  if (pools.size() > 4) return fail(SA_ERR_UNSUPPORTED, "more than 4 granularities");
  sa::DecodeScoreParams dp{};
  std::memset(&dp, 0, sizeof dp);
  dp.q = q;
  dp.qs0 = desc->q_stride[0];
  dp.qs1 = desc->q_stride[1];
  dp.pooled = pooled;
  {
    int64_t off = 0;
    for (size_t i = 0; i < pools.size(); ++i) {
      dp.pool_off[i] = off;
      dp.pool_nc[i] = int(cdiv(desc->kv_len, pools[i]));
      off += int64_t(pooled_elems(desc, pools[i]));
    }
  }
  dp.s = sc;
  dp.nc_max = w.nc_max;
  dp.Hq = desc->n_q_heads;
  dp.Hkv = desc->n_kv_heads;
  // short streams: many waves balance better than long ones; 32 rows are the
  // four 8-row stages of a wave's ring, three of them issued at once (a sweep
  // of the 128K decode step: 32 rows 212.5-214.4 us, 48 214.9-216.1, 64
  // 215.3-219.5, 40 215.7-217.3, 24 219.6-220.2, 128 218.8-220.4, 16 226.9-229.0)
  dp.rows_per_wg = 32;
  dp.scale = scale;
  // jobs: (KV head, granularity) -> the scoring heads, at most 8 per job
  std::vector<sa::DecodeScoreJob> jobs;
  for (int j = 0; j < desc->n_kv_heads; ++j)
    for (size_t pi = 0; pi < pools.size(); ++pi) {
      sa::DecodeScoreJob job;
      std::memset(&job, 0, sizeof job);
      job.kvh = j;
      job.pool = int(pi);
      for (int gi = 0; gi < G; ++gi) {
        const int h = j * G + gi;
        if (decode_scores_head(desc, budgets[h]) && budgets[h].granularity == pools[pi]) {
          if (job.n_heads == 8) {
            jobs.push_back(job);
            job.n_heads = 0;
          }
          job.heads[job.n_heads++] = h;
        }
      }
      if (job.n_heads) jobs.push_back(job);
    }
  for (size_t j0 = 0; j0 < jobs.size(); j0 += sa::kMaxScoreJobs) {
    const size_t nj = std::min<size_t>(sa::kMaxScoreJobs, jobs.size() - j0);
    dp.n_jobs = int(nj);
    for (size_t i = 0; i < nj; ++i) dp.jobs[i] = jobs[j0 + i];
    if ((e = sa::launch_decode_scores(dp, desc->dtype, D, desc->batch, st)) != hipSuccess)
      return hip_fail(e, "decode scores");
  }
  tp.s = sc;
  tp.s_row = w.nc_max;
  tp.rows = desc->batch * desc->n_q_heads;
  tp.kv_len = desc->kv_len;
  if ((e = sa::launch_topk(tp, w.nc_max, st)) != hipSuccess) return hip_fail(e, "decode top-k");
  return ok();
}

size_t sa_prefill_workspace_size(const sa_attn_desc* desc, int32_t kmax, int32_t n_bins) {
  (void)desc;
  (void)kmax;
  (void)n_bins;
  return 256;  // the work-queue counter
}

static sa_status prefill_impl(const sa_attn_desc* desc, const void* q, const void* k, const void* v, void* o,
                              float* lse, const int32_t* block_idx, const int32_t* block_cnt, int32_t kmax,
                              const float* key_norms, const int32_t* bin_offsets, const int32_t* items_by_bin, int32_t n_bins,
                              const int32_t* queue_offsets, int32_t n_queues, int32_t out_f32, void* workspace,
                              size_t workspace_bytes, void* stream, uint64_t* wg_times = nullptr) {
  sa_status s = check_desc(desc, true);
  if (s) return s;
  if (!q || !k || !v || !o || !block_idx || !block_cnt) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SA_ERR_INVALID_ARG, "q, k, v, o must be 16-byte aligned");
  if (kmax < 1) return fail(SA_ERR_INVALID_ARG, "kmax must be >= 1");
  if (reinterpret_cast<uintptr_t>(key_norms) & 3) return fail(SA_ERR_INVALID_ARG, "key_norms must be 4-byte aligned");
  if (bin_offsets && !items_by_bin) return fail(SA_ERR_INVALID_ARG, "bin_offsets without items_by_bin");
  if (items_by_bin && n_bins < 1) return fail(SA_ERR_INVALID_ARG, "n_bins must be >= 1");
  const bool queue = items_by_bin && !bin_offsets;
  if (queue && (!workspace || workspace_bytes < size_t(4) * n_queues || (reinterpret_cast<uintptr_t>(workspace) & 3)))
    return fail(SA_ERR_INVALID_ARG, "the work queue needs a 4-byte aligned workspace of >= %d bytes", 4 * n_queues);
  if (desc->batch >= 32768 || desc->n_kv_heads >= 65536)
    return fail(SA_ERR_UNSUPPORTED, "batch must be < 32768 and n_kv_heads < 65536");
  const int64_t nb = cdiv(desc->q_len, desc->block_size);
  const int64_t n_tiles = int64_t(desc->batch) * desc->n_q_heads * nb;
  if (n_tiles > (1ll << 30)) return fail(SA_ERR_UNSUPPORTED, "too many tiles");
  if (queue_offsets) {
    if (queue_offsets[0] != 0 || queue_offsets[n_queues] != n_tiles)
      return fail(SA_ERR_INVALID_ARG, "queue_offsets must run from 0 to the tile count %lld", (long long)n_tiles);
    for (int32_t i = 0; i < n_queues; ++i)
      if (queue_offsets[i + 1] < queue_offsets[i]) return fail(SA_ERR_INVALID_ARG, "queue_offsets must not decrease");
  }
  {
    const int64_t es = elem_size(desc->dtype);
    if (int64_t(desc->kv_len + 256) * desc->k_stride[2] * es >= (1ll << 31) ||
        int64_t(desc->kv_len + 256) * desc->v_stride[2] * es >= (1ll << 31))
      return fail(SA_ERR_UNSUPPORTED, "one (batch, KV head) slice of K or V must span < 2 GiB");
  }
  if ((s = check_device())) return s;
  sa::PrefillParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.qs0 = desc->q_stride[0];
  p.qs1 = desc->q_stride[1];
  p.qs2 = desc->q_stride[2];
  p.ks0 = desc->k_stride[0];
  p.ks1 = desc->k_stride[1];
  p.ks2 = desc->k_stride[2];
  p.vs0 = desc->v_stride[0];
  p.vs1 = desc->v_stride[1];
  p.vs2 = desc->v_stride[2];
  p.os0 = desc->o_stride[0];
  p.os1 = desc->o_stride[1];
  p.os2 = desc->o_stride[2];
  p.block_idx = block_idx;
  p.block_cnt = block_cnt;
  p.kmax = kmax;
  p.bin_offsets = bin_offsets;
  p.items_by_bin = items_by_bin;
  p.Hq = desc->n_q_heads;
  p.G = desc->n_q_heads / desc->n_kv_heads;
  p.S = desc->q_len;
  p.NB = int(nb);
  p.n_tiles = int(n_tiles);
  p.scale_log2 = scale_of(desc) * 1.4426950408889634f;
  p.out_f32 = out_f32 ? 1 : 0;
  p.queue = queue ? static_cast<int*>(workspace) : nullptr;
  p.n_queues = n_queues;
  for (int32_t i = 0; i <= n_queues; ++i) p.qoff[i] = queue_offsets ? queue_offsets[i] : (i ? int(n_tiles) : 0);
  if (wg_times && (reinterpret_cast<uintptr_t>(wg_times) & 7))
    return fail(SA_ERR_INVALID_ARG, "wg_times must be 8-byte aligned");
  p.wg_times = wg_times;
  p.key_norms = key_norms;
  if (debug_checks((hipStream_t)stream)) {
    const int NB = int(nb);
    if ((s = check_lists(block_idx, block_cnt, n_tiles, kmax, [NB](int64_t t) { return int32_t(t % NB) + 1; },
                         (hipStream_t)stream, "prefill")))
      return s;
    if (items_by_bin && (s = check_items(items_by_bin, bin_offsets, n_bins, n_tiles, (hipStream_t)stream))) return s;
    if (key_norms && (s = check_key_norms(desc, k, key_norms, (hipStream_t)stream))) return s;
  }
  const int grid = items_by_bin ? n_bins : int(n_tiles);
  hipError_t e = sa::launch_prefill(p, desc->dtype, desc->head_dim, desc->block_size, desc->kernel_variant, grid,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
  return ok();
}

sa_status sa_sparse_attn_prefill(const sa_attn_desc* desc, const void* q, const void* k, const void* v, void* o,
                                 float* lse, const int32_t* block_idx, const int32_t* block_cnt, int32_t kmax,
                                 const float* key_norms, const int32_t* bin_offsets, const int32_t* items_by_bin,
                                 int32_t n_bins, int32_t out_f32, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return prefill_impl(desc, q, k, v, o, lse, block_idx, block_cnt, kmax, key_norms, bin_offsets, items_by_bin, n_bins,
                      nullptr, 1, out_f32, workspace, workspace_bytes, stream);
}

sa_status sa_sparse_attn_prefill_queues(const sa_attn_desc* desc, const void* q, const void* k, const void* v,
                                        void* o, float* lse, const int32_t* block_idx, const int32_t* block_cnt,
                                        int32_t kmax, const float* key_norms, const int32_t* queue_offsets,
                                        int32_t n_queues,
                                        const int32_t* order, int32_t n_workgroups, int32_t out_f32, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (n_queues < 1 || n_queues > kMaxQueues)
    return fail(SA_ERR_INVALID_ARG, "n_queues %d outside [1, %d]", n_queues, kMaxQueues);
  if (!queue_offsets || !order) return fail(SA_ERR_INVALID_ARG, "queue_offsets or order is NULL");
  return prefill_impl(desc, q, k, v, o, lse, block_idx, block_cnt, kmax, key_norms, nullptr, order, n_workgroups,
                      queue_offsets, n_queues, out_f32, workspace, workspace_bytes, stream);
}

sa_status sa_sparse_attn_prefill_timed(const sa_attn_desc* desc, const void* q, const void* k, const void* v,
                                       void* o, float* lse, const int32_t* block_idx, const int32_t* block_cnt,
                                       int32_t kmax, const float* key_norms, const int32_t* bin_offsets, const int32_t* items_by_bin,
                                       int32_t n_bins, const int32_t* queue_offsets, int32_t n_queues,
                                       int32_t out_f32, uint64_t* wg_times, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!wg_times) return fail(SA_ERR_INVALID_ARG, "wg_times is NULL");
  if (queue_offsets) {
    if (n_queues < 1 || n_queues > kMaxQueues)
      return fail(SA_ERR_INVALID_ARG, "n_queues %d outside [1, %d]", n_queues, kMaxQueues);
    if (!items_by_bin || bin_offsets) return fail(SA_ERR_INVALID_ARG, "queues need items_by_bin and no bin_offsets");
  } else {
    n_queues = 1;
  }
  return prefill_impl(desc, q, k, v, o, lse, block_idx, block_cnt, kmax, key_norms, bin_offsets, items_by_bin, n_bins,
                      queue_offsets, n_queues, out_f32, workspace, workspace_bytes, stream, wg_times);
}

size_t sa_decode_workspace_size(const sa_attn_desc* desc, const sa_head_budget* budgets, int32_t kmax) {
  (void)kmax;
  if (check_desc(desc, false) || check_budgets(desc, budgets, false)) return 0;
  return decode_attn_ws(desc, budgets).total;
}

static sa_status decode_impl(const sa_attn_desc* desc, const sa_head_budget* budgets, const void* q, const void* k,
                             const void* v, const sa_kv_pages* pages, void* o, float* lse, const int32_t* block_idx,
                             const int32_t* block_cnt, int32_t kmax, int32_t out_f32, void* workspace,
                             size_t workspace_bytes, void* stream) {
  sa_status s = check_desc(desc, false);
  if (s) return s;
  if ((s = check_budgets(desc, budgets, false))) return s;
  if (pages) {
    if ((s = check_pages(desc, pages))) return s;
    if (desc->dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "paged caches are supported for bf16 only");
  }
  if (!q || !k || !v || !o || !block_idx || !block_cnt) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(k) || !aligned16(v)) return fail(SA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  const int G = desc->n_q_heads / desc->n_kv_heads;
  if (G > 8) return fail(SA_ERR_UNSUPPORTED, "GQA group size %d > 8", G);
  int32_t need = 0;
  sa_decode_block_counts(desc, budgets, nullptr, &need);
  if (kmax < need) return fail(SA_ERR_INVALID_ARG, "kmax %d < largest block count %d", kmax, need);
  const DecodeAttnWs w = decode_attn_ws(desc, budgets);
  if (!workspace || workspace_bytes < w.total)
    return fail(SA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total, workspace_bytes);
  if (!aligned16(workspace)) return fail(SA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const int64_t n_atoms = cdiv(desc->kv_len, sa::kAtom);
  if (int64_t(G) * cdiv(n_atoms, 32) * 4 > 64 * 1024) return fail(SA_ERR_UNSUPPORTED, "kv_len too long for the plan");
  if (!pages) {
    // the attention kernels address a (sequence, KV head) slice with 32-bit offsets
    const int64_t es = elem_size(desc->dtype);
    if (int64_t(desc->kv_len + kAtomPad) * desc->k_stride[2] * es >= (1ll << 31) ||
        int64_t(desc->kv_len + kAtomPad) * desc->v_stride[2] * es >= (1ll << 31))
      return fail(SA_ERR_UNSUPPORTED, "one (sequence, KV head) slice of K or V must span < 2 GiB");
  }
  if ((s = check_device())) return s;
  hipStream_t st = (hipStream_t)stream;
  if (debug_checks(st)) {
    const int Hq = desc->n_q_heads, L = desc->kv_len;
    if ((s = check_lists(block_idx, block_cnt, int64_t(desc->batch) * Hq, kmax,
                         [&](int64_t r) { return int32_t(cdiv(L, budgets[r % Hq].granularity)); }, st, "decode")))
      return s;
    if (pages && (s = check_table(desc, pages, st))) return s;
  }
  char* ws = static_cast<char*>(workspace);
  uint32_t* atoms = reinterpret_cast<uint32_t*>(ws + w.atoms);
  int32_t* n_union = reinterpret_cast<int32_t*>(ws + w.n_union);
  float* part_o = reinterpret_cast<float*>(ws + w.part_o);
  float* part_ml = reinterpret_cast<float*>(ws + w.part_ml);
  hipError_t e;
  sa::DecodePlanParams pp{};
  pp.block_idx = block_idx;
  pp.block_cnt = block_cnt;
  pp.kmax = kmax;
  pp.Hq = desc->n_q_heads;
  pp.Hkv = desc->n_kv_heads;
  pp.G = G;
  pp.kv_len = desc->kv_len;
  pp.n_atoms = int(n_atoms);
  pp.max_union = w.max_union;
  pp.atoms = atoms;
  pp.n_union = n_union;
  pp.heads = make_table(desc, budgets, false);
  if ((e = sa::launch_decode_plan(pp, desc->batch, st)) != hipSuccess) return hip_fail(e, "decode plan");
  sa::DecodeAttnParams ap{};
  ap.q = q;
  ap.qs0 = desc->q_stride[0];
  ap.qs1 = desc->q_stride[1];
  ap.k = k;
  ap.v = v;
  ap.ks0 = desc->k_stride[0];
  ap.ks1 = desc->k_stride[1];
  ap.ks2 = desc->k_stride[2];
  ap.vs0 = desc->v_stride[0];
  ap.vs1 = desc->v_stride[1];
  ap.vs2 = desc->v_stride[2];
  ap.atoms = atoms;
  ap.n_union = n_union;
  ap.max_union = w.max_union;
  ap.chunk_atoms = kChunkAtoms;
  ap.n_chunks = w.n_chunks;
  ap.Hq = desc->n_q_heads;
  ap.Hkv = desc->n_kv_heads;
  ap.G = G;
  ap.kv_len = desc->kv_len;
  ap.scale_log2 = scale_of(desc) * 1.4426950408889634f;
  ap.pages = page_table_of(pages);
  ap.part_o = part_o;
  ap.part_ml = part_ml;
  if ((e = sa::launch_decode_attn(ap, desc->dtype, desc->head_dim, desc->batch, st)) != hipSuccess)
    return hip_fail(e, "decode attention");
  sa::DecodeCombineParams cp{};
  cp.part_o = part_o;
  cp.part_ml = part_ml;
  cp.n_union = n_union;
  cp.chunk_atoms = kChunkAtoms;
  cp.n_chunks = w.n_chunks;
  cp.Hq = desc->n_q_heads;
  cp.Hkv = desc->n_kv_heads;
  cp.G = G;
  cp.o = o;
  cp.os0 = desc->o_stride[0];
  cp.os1 = desc->o_stride[1];
  cp.lse = lse;
  cp.out_f32 = out_f32 ? 1 : 0;
  if ((e = sa::launch_decode_combine(cp, desc->dtype, desc->head_dim, desc->batch, st)) != hipSuccess)
    return hip_fail(e, "decode combine");
  return ok();
}

sa_status sa_block_attention_mass(const sa_attn_desc* desc, const void* q, const void* k, float* mass,
                                  void* stream) {
  sa_status s = check_desc(desc, true);
  if (s) return s;
  if (desc->dtype != SA_BF16 || desc->block_size != 128)
    return fail(SA_ERR_UNSUPPORTED, "block attention mass needs bf16 inputs and block_size 128");
  if (!q || !k || !mass) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(mass) & 3))
    return fail(SA_ERR_INVALID_ARG, "q and k must be 16-byte aligned, mass 4-byte aligned");
  if ((s = check_device())) return s;
  sa::MassParams p{};
  p.q = q;
  p.k = k;
  p.qs0 = desc->q_stride[0];
  p.qs1 = desc->q_stride[1];
  p.qs2 = desc->q_stride[2];
  p.ks0 = desc->k_stride[0];
  p.ks1 = desc->k_stride[1];
  p.ks2 = desc->k_stride[2];
  p.mass = mass;
  p.Hq = desc->n_q_heads;
  p.G = desc->n_q_heads / desc->n_kv_heads;
  p.S = desc->q_len;
  p.NB = int(cdiv(desc->q_len, 128));
  p.scale_log2 = scale_of(desc) * 1.4426950408889634f;
  const hipError_t e = sa::launch_block_mass(p, desc->head_dim, desc->batch, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "block attention mass");
  return ok();
}

sa_status sa_output_deviation(const sa_attn_desc* desc, const float* o_approx, const float* o_ref, double* dev,
                              void* stream) {
  sa_status s = check_desc(desc, true);
  if (s) return s;
  if (!o_approx || !o_ref || !dev) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned16(o_approx) || !aligned16(o_ref) || (reinterpret_cast<uintptr_t>(dev) & 7))
    return fail(SA_ERR_INVALID_ARG, "o_approx and o_ref must be 16-byte aligned, dev 8-byte aligned");
  if (desc->head_dim % 4 || desc->o_stride[0] % 4 || desc->o_stride[1] % 4 || desc->o_stride[2] % 4)
    return fail(SA_ERR_INVALID_ARG, "head_dim and the o strides must be multiples of 4 elements");
  if ((s = check_device())) return s;
  sa::DeviationParams p{};
  p.a = o_approx;
  p.r = o_ref;
  p.s0 = desc->o_stride[0];
  p.s1 = desc->o_stride[1];
  p.s2 = desc->o_stride[2];
  p.batch = desc->batch;
  p.Hq = desc->n_q_heads;
  p.S = desc->q_len;
  p.D = desc->head_dim;
  p.dev = dev;
  const hipError_t e = sa::launch_output_deviation(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "output deviation");
  return ok();
}

sa_status sa_budget_recovery(const float* mass, int32_t batch, int32_t n_heads, int32_t n_blocks,
                             const sa_head_budget* budgets, int32_t step_q16, double* recovery) {
  if (!mass || !budgets || !recovery) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (batch < 1 || n_heads < 1 || n_blocks < 1) return fail(SA_ERR_INVALID_ARG, "batch, n_heads, n_blocks must be >= 1");
  if (step_q16 < 1 || 65536 % step_q16) return fail(SA_ERR_INVALID_ARG, "step_q16 %d must divide 65536", step_q16);
  for (int32_t h = 0; h < n_heads; ++h) {
    const sa_head_budget& b = budgets[h];
    if (b.n_sink < 0 || b.n_local < 0 || b.min_blocks < b.n_sink + b.n_local || b.min_blocks < 1)
      return fail(SA_ERR_INVALID_ARG, "head %d: need min_blocks >= max(1, n_sink + n_local)", h);
  }
  const int32_t n_grid = 65536 / step_q16;
  std::vector<int32_t> order, rank(n_blocks);
  std::vector<char> forced(n_blocks);
  for (int32_t h = 0; h < n_heads; ++h) {
    const sa_head_budget& bud = budgets[h];
    std::vector<double> acc(n_grid, 0.0);
    for (int32_t bi = 0; bi < batch; ++bi) {
      for (int32_t m = 0; m < n_blocks; ++m) {
        const float* w = mass + (((int64_t)bi * n_heads + h) * n_blocks + m) * n_blocks;
        const int32_t nc = m + 1;
        // ranking: the forced blocks, then the others heaviest first, ties to the lowest index
        order.clear();
        int32_t n_forced = 0;
        for (int32_t n = 0; n < nc; ++n) {
          forced[n] = n < bud.n_sink || n >= nc - bud.n_local;
          if (forced[n]) {
            order.push_back(n);
            ++n_forced;
          }
        }
        for (int32_t n = 0; n < nc; ++n)
          if (!forced[n]) order.push_back(n);
        std::stable_sort(order.begin() + n_forced, order.end(),
                         [&](int32_t a, int32_t b) { return double(w[a]) > double(w[b]); });
        for (int32_t r = 0; r < nc; ++r) rank[order[r]] = r;
        double total = 0.0;
        for (int32_t n = 0; n < nc; ++n) total += double(w[n]);
        for (int32_t i = 0; i < n_grid; ++i) {
          const int32_t kk = sa::budget_blocks(nc, bud.min_blocks, uint32_t((i + 1) * step_q16));
          double kept = 0.0;
          for (int32_t n = 0; n < nc; ++n)
            if (rank[n] < kk) kept += double(w[n]);
          acc[i] += total > 0.0 ? kept / total : 1.0;
        }
      }
    }
    for (int32_t i = 0; i < n_grid; ++i) recovery[(int64_t)h * n_grid + i] = acc[i] / (double(batch) * n_blocks);
  }
  return ok();
}

sa_status sa_budget_shift(const double* recovery, int32_t n_heads, int32_t step_q16, int64_t total_q16,
                          uint32_t* ratio_q16) {
  if (!recovery || !ratio_q16) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (n_heads < 1) return fail(SA_ERR_INVALID_ARG, "n_heads must be >= 1");
  if (step_q16 < 1 || 65536 % step_q16) return fail(SA_ERR_INVALID_ARG, "step_q16 %d must divide 65536", step_q16);
  const int64_t per = total_q16 / n_heads;
  if (per * n_heads != total_q16 || per % step_q16 || per < step_q16 || per > 65536)
    return fail(SA_ERR_INVALID_ARG, "total_q16 must be n_heads times a whole number of steps in [step, 65536]");
  const int32_t n_grid = 65536 / step_q16;
  auto rec = [&](int32_t h, int32_t i) { return recovery[(int64_t)h * n_grid + i]; };
  std::vector<int32_t> idx(n_heads, int32_t(per / step_q16) - 1);
  while (true) {
    int32_t b = -1;
    for (int32_t h = 0; h < n_heads; ++h)
      if (idx[h] + 1 < n_grid && (b < 0 || rec(h, idx[h]) < rec(b, idx[b]))) b = h;
    if (b < 0) break;
    int32_t a = -1;
    for (int32_t h = 0; h < n_heads; ++h)
      if (h != b && idx[h] >= 1 && (a < 0 || rec(h, idx[h] - 1) > rec(a, idx[a] - 1))) a = h;
    if (a < 0 || !(rec(a, idx[a] - 1) > rec(b, idx[b]))) break;
    --idx[a];
    ++idx[b];
  }
  for (int32_t h = 0; h < n_heads; ++h) ratio_q16[h] = uint32_t((idx[h] + 1) * step_q16);
  return ok();
}

sa_status sa_sparse_attn_decode(const sa_attn_desc* desc, const sa_head_budget* budgets, const void* q,
                                const void* k, const void* v, void* o, float* lse, const int32_t* block_idx,
                                const int32_t* block_cnt, int32_t kmax, int32_t out_f32, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return decode_impl(desc, budgets, q, k, v, nullptr, o, lse, block_idx, block_cnt, kmax, out_f32, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free decode
// The scratch of sa_sparse_attn_decode_noalloc: one fixed array in device
// memory per GPU, held from the loading of this library's code object on that
// GPU until the process ends.  In host code the name is only a host-side
// stand-in: the device address comes from hipGetSymbolAddress, once per device
// (with that device current), and only that address is handed to kernels.
static __device__ __align__(256) char scratch[SA_DECODE_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first
// call on that device).
sa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_NO_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}
}  // namespace

extern "C" {

sa_status sa_sparse_attn_decode_noalloc(const sa_attn_desc* desc, const sa_head_budget* budgets, const void* q,
                                        const void* k, const void* v, void* o, float* lse,
                                        const int32_t* block_idx, const int32_t* block_cnt, int32_t kmax,
                                        int32_t out_f32, void* stream) {
  sa_status s = check_desc(desc, false);
  if (s) return s;
  if ((s = check_budgets(desc, budgets, false))) return s;
  const size_t need = decode_attn_ws(desc, budgets).total;
  if (need > size_t(SA_DECODE_SCRATCH_BYTES))
    return fail(SA_ERR_WORKSPACE, "decode needs %zu bytes of scratch, the fixed array holds %zu", need,
                size_t(SA_DECODE_SCRATCH_BYTES));
  if ((s = check_device())) return s;
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws))) return s;
  // nothing in the scratch has to start at zero: the plan kernel writes every
  // atom list and count the attention reads, and every chunk partial is
  // written before the combine reads it
  return decode_impl(desc, budgets, q, k, v, nullptr, o, lse, block_idx, block_cnt, kmax, out_f32, ws,
                     size_t(SA_DECODE_SCRATCH_BYTES), stream);
}

sa_status sa_sparse_attn_decode_paged(const sa_attn_desc* desc, const sa_head_budget* budgets, const void* q,
                                      const void* k_pages, const void* v_pages, const sa_kv_pages* pages, void* o,
                                      float* lse, const int32_t* block_idx, const int32_t* block_cnt, int32_t kmax,
                                      int32_t out_f32, void* workspace, size_t workspace_bytes, void* stream) {
  if (!pages) return fail(SA_ERR_INVALID_ARG, "pages is NULL");
  return decode_impl(desc, budgets, q, k_pages, v_pages, pages, o, lse, block_idx, block_cnt, kmax, out_f32,
                     workspace, workspace_bytes, stream);
}


sa_status sa_measure_mfma_peak(int32_t n_workgroups, int32_t iters, int32_t operands, float* sink, void* stream) {
  if (!sink) return fail(SA_ERR_INVALID_ARG, "sink is NULL");
  if (operands != 0 && operands != 1) return fail(SA_ERR_INVALID_ARG, "operands %d is not 0 (ones) or 1 (random)", operands);
  if (n_workgroups < 1 || n_workgroups > (1 << 20)) return fail(SA_ERR_INVALID_ARG, "n_workgroups %d out of [1, 2^20]", n_workgroups);
  if (iters < 1 || iters > 65536) return fail(SA_ERR_INVALID_ARG, "iters %d out of [1, 65536]", iters);
  if (reinterpret_cast<uintptr_t>(sink) & 3) return fail(SA_ERR_INVALID_ARG, "sink must be 4-byte aligned");
  sa_status s = check_device();
  if (s) return s;
  const hipError_t e = sa::launch_mfma_peak(n_workgroups, iters, operands == 1, sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mfma peak");
  return ok();
}

sa_status sa_measure_hbm_read(const void* buf, int64_t bytes, int32_t n_workgroups, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(SA_ERR_INVALID_ARG, "NULL pointer");
  if (bytes < 16 || bytes % 16) return fail(SA_ERR_INVALID_ARG, "bytes %lld must be a positive multiple of 16", (long long)bytes);
  if (n_workgroups < 1 || n_workgroups > (1 << 20)) return fail(SA_ERR_INVALID_ARG, "n_workgroups %d out of [1, 2^20]", n_workgroups);
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(SA_ERR_INVALID_ARG, "buf must be 16-byte aligned, sink 4-byte aligned");
  sa_status s = check_device();
  if (s) return s;
  const hipError_t e = sa::launch_hbm_read(buf, bytes, sink, n_workgroups, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hbm read");
  return ok();
}

}  // extern "C"
