// The step cursor of the persistent prefill attention kernels: which tile
// (batch, query head, query block) a workgroup works on and which 64-key step
// of which selected key block comes next.
//
// Work order (the greedy longest-load-first schedule of "S-HPLB: Efficient LLM
// Attention Serving via Sparsity-Aware Head Parallelism Load Balance", Italian
// summary §2.B / Chinese summary §2.2, applied on one GPU):
//   * work queue (p.queue set): the workgroups take the items of one global
//     list in order, each claiming its next item from a counter when it starts
//     the current one, so faster compute units simply take more items.  The
//     list may be cut into partitions with one counter each (one per XCD, so
//     the workgroups of an XCD share its L2): a workgroup starts on partition
//     blockIdx.x % n_queues and, once that is empty, moves on to the following
//     ones in turn; after trying every partition it is done.  Wave 0 makes the
//     claims and hands each to the other waves through LDS;
//   * static bins (p.bin_offsets set): workgroup w walks items
//     [bin_offsets[w], bin_offsets[w+1]) of items_by_bin;
//   * natural grid: workgroup w runs tile w.
// The item list and each tile's block list are read through per-wave register
// windows (lane l holds entry base + l) and picked out with readlane, so
// advancing a step never waits on memory; the first window of the next item's
// blocks is fetched while the current item runs.
#pragma once

#include "sa_prefill_common.hpp"

namespace sa {
namespace prefill {

// LDS state of the queue claims, shared by the waves of a workgroup.
struct QueueLds {
  int slot;      // position handed from wave 0 to the others
  int state[2];  // wave 0: current partition, partitions left to try
};

template <int kNSub>  // 64-key steps per key block
struct Cursor {
  QueueLds* q;
  int wave, lane;
  bool qmode;
  int it_end;
  int q_pend = 0;                           // wave 0, lane 0: the claim in flight
  int ibase = 0, iw_tile = -1, iw_cnt = 0;  // per lane: tile and block count of item ibase + lane
  int c_cnt = 0, c_wbase = 0, c_win = -1;   // blocks of the cursor's tile: window at c_wbase
  int nx_item = -1, nx_win = -1;            // prefetched first window of item nx_item
  int nx_tile = -1, nx_cnt = 0;             // queue mode: its tile and block count
  int q_next = 0;                           // queue mode: the item after the cursor's
  Step cur;

  __device__ __forceinline__ void claim() {
    if (wave == 0 && lane == 0 && q->state[1] > 0) q_pend = atomicAdd(COLD(queue) + q->state[0], 1);
  }
  // position in items_by_bin of the claim in flight (n_tiles: none left)
  __device__ __forceinline__ int take_claim() {
    __syncthreads();  // every wave has read the previous claim
    if (wave == 0) {
      const int n_tiles = COLD(n_tiles), nq = COLD(n_queues);
      int qc = __builtin_amdgcn_readfirstlane(q->state[0]);
      int left = __builtin_amdgcn_readfirstlane(q->state[1]);
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
        q->slot = pos;
        q->state[0] = qc;
        q->state[1] = left;
      }
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(q->slot);
  }

  // first item of this workgroup; sets the mode and it_end
  __device__ __forceinline__ int begin(QueueLds* lds, int wave_, int lane_) {
    q = lds;
    wave = wave_;
    lane = lane_;
    qmode = COLD(queue) != nullptr;
    cur.valid = 0;
    int it_beg;
    if (qmode) {
      if (wave == 0 && lane == 0) {
        q->state[0] = blockIdx.x % COLD(n_queues);
        q->state[1] = COLD(n_queues);
      }
      claim();
      it_beg = take_claim();
      claim();
      it_end = COLD(n_tiles);  // positions in the global list
    } else if (COLD(bin_offsets)) {
      it_beg = COLD(bin_offsets)[blockIdx.x];
      it_end = COLD(bin_offsets)[blockIdx.x + 1];
    } else {
      it_beg = blockIdx.x;
      it_end = (int)blockIdx.x < COLD(n_tiles) ? (int)blockIdx.x + 1 : (int)blockIdx.x;
    }
    load_items(it_beg);
    cur.item = -1;
    seek(it_beg, 0);
    return it_beg;
  }

  __device__ __forceinline__ void load_items(int base) {
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
  }
  __device__ __forceinline__ int load_blocks(int tile, int cnt, int base) {
    const int jj = base + lane;
    return jj < cnt ? COLD(block_idx)[(int64_t)tile * COLD(kmax) + jj] : -1;
  }
  // queue mode: tile and block count of the item at position it
  __device__ __forceinline__ void queue_item(int it, int& tile, int& cnt) {
    tile = COLD(items_by_bin)[it];
    if (tile >= 0 && tile < COLD(n_tiles)) {
      cnt = min(COLD(block_cnt)[tile], COLD(kmax));
    } else {
      tile = -1;
      cnt = 0;
    }
  }
  __device__ __forceinline__ void item_tile(int it, int& tile, int& cnt) {
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
  }
  __device__ __forceinline__ void prefetch_next(int it) {
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
  }
  // first valid block at or after position j of item `it` (moving to later items)
  __device__ __forceinline__ void seek(int it, int j) {
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
          cur.kvs = ((cur.bh / Hq) << 16) | ((cur.bh % Hq) / COLD(G));
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
  }
  __device__ __forceinline__ void advance() {
    if (!cur.valid) return;
    if (cur.hs + 1 < kNSub) {
      cur.hs += 1;
      return;
    }
    seek(cur.item, cur.j + 1);
  }
};

}  // namespace prefill
}  // namespace sa
