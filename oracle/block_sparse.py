"""fp64 CPU oracle: per-head-budget block-sparse attention, written from the pages.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Every function here is a
plain, slow, obviously-correct statement of one step of the method.  Floating
point is fp64 throughout; bf16 inputs arrive as raw uint16 bit patterns and are
widened exactly.  Library primitives used as single steps: ``numpy`` matmul,
``exp``, ``log``, ``argsort``-free Python sorting, ``heapq``.

Sources (gist.science technical summaries):
  * "S-HPLB: Efficient LLM Attention Serving via Sparsity-Aware Head Parallelism
    Load Balance" -- Italian summary ("Sommario tecnico") and Chinese summary
    ("技术摘要").  Per-head budgets (§2.A / §2.1), top-k sparse attention (§1),
    greedy longest-budget-first placement (§2.B / §2.2).
  * "Fluxion" -- Italian technical summary, "Intuizioni Chiave" 2 (block
    granularity, streaming vs retrieval heads) and "Componenti di Sistema"
    (GQA group-level data volume).
  * "Unifying Sparse Attention with Hierarchical Memory for Scalable
    Long-Context LLM Serving" (Spin) -- Spanish summary §2.A (Index / Select /
    Attention operations).

Where the pages leave a step open the plainest reading is taken; each reading is
named in the docstring of the function that applies it (R-numbers refer to the
list of readings kept with the design notes).

Parity status: every function below is pinned by tests in ``tests/`` against
closed forms, textbook routines or brute force; none is "parity unpinned".
"""

from __future__ import annotations

import heapq
import itertools
import math
from typing import Mapping, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# input widening
# ----------------------------------------------------------------------------


def to_f64(x: np.ndarray) -> np.ndarray:
    """Widen an input tensor to fp64 exactly.

    ``uint16`` arrays are bf16 bit patterns: a bf16 value is the fp32 value whose
    upper 16 bits are the pattern and whose lower 16 bits are zero.  ``float32``
    and ``float64`` arrays are widened as they are.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


# ----------------------------------------------------------------------------
# O1  pooling  (Spin summary §2.A, "Index"; block granularity: Fluxion summary,
#     Intuizioni Chiave 2)
# ----------------------------------------------------------------------------


def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of the rows of each block of ``block`` consecutive tokens.

    ``x[..., T, D]`` -> ``[..., ceil(T/block), D]``.  A short last block (``T``
    not a multiple of ``block``) is averaged over the rows it has.  Reading R1:
    a query block is represented by the mean of its query rows, the same
    operator as for keys.
    """
    if block <= 0:
        raise ValueError("block must be positive")
    T = x.shape[-2]
    nb = -(-T // block)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]), dtype=np.float64)
    for n in range(nb):
        lo, hi = n * block, min(T, (n + 1) * block)
        rows = to_f64(x[..., lo:hi, :])
        out[..., n, :] = rows.sum(axis=-2) / float(hi - lo)
    return out


# ----------------------------------------------------------------------------
# O3  budget rule  (S-HPLB summaries: per-head budget fixed offline, §2.A / §2.1;
#     the stable quantity is the per-head budget *ratio*, Chinese §2.1)
# ----------------------------------------------------------------------------


def budget_blocks(n_cand: int, min_blocks: int, ratio_q16: int) -> int:
    """Number of key blocks a row keeps, in exact integer arithmetic.

    ``k = min(n_cand, max(min_blocks, ceil(ratio_q16 * n_cand / 65536)))``.
    Readings R3/R4: a head's budget is a ratio of the blocks it may see
    (``ratio_q16`` in units of 2**-16, zero for a fixed count) with a floor of
    ``min_blocks``; the forced blocks count against it (R5).
    """
    n_cand, min_blocks, ratio_q16 = int(n_cand), int(min_blocks), int(ratio_q16)
    want = max(min_blocks, (ratio_q16 * n_cand + 65535) // 65536)
    return min(n_cand, want)


def forced_blocks(n_cand: int, n_sink: int, n_local: int) -> list[int]:
    """Blocks always kept: the first ``n_sink`` and the last ``n_local`` of the
    ``n_cand`` candidates (sink and local blocks; Fluxion summary, Intuizioni
    Chiave 1-2: attention-sink tokens and streaming heads)."""
    f = set(range(min(n_sink, n_cand))) | set(range(max(0, n_cand - n_local), n_cand))
    return sorted(f)


# ----------------------------------------------------------------------------
# O4  top-k selection (S-HPLB summaries §1: a top-k token budget per head)
# ----------------------------------------------------------------------------


def select_row(scores: Sequence[float], k: int, n_sink: int, n_local: int) -> list[int]:
    """Blocks kept by one row: the forced set plus the best ``k - |F|`` others.

    Others are ranked by score, highest first, ties to the lowest block index
    (reading R8; -0.0 and +0.0 compare equal).  Returned in ascending order.
    A plain full sort of the candidates -- brute force by construction.
    """
    n = len(scores)
    F = forced_blocks(n, n_sink, n_local)
    if k < len(F) or k > n:
        raise ValueError(f"budget {k} outside [{len(F)}, {n}]")
    fs = set(F)
    rest = [i for i in range(n) if i not in fs]
    rest.sort(key=lambda i: (-float(scores[i]), i))
    return sorted(F + rest[: k - len(F)])


# ----------------------------------------------------------------------------
# O2 + O4 for prefill
# ----------------------------------------------------------------------------


def prefill_block_scores(q, k, block: int, scale: float | None = None) -> np.ndarray:
    """Block scores ``s[b,h,m,n] = scale * <mean Q block m of head h, mean K
    block n of KV head h // G>`` for ``n <= m``; ``-inf`` above the diagonal.

    q: ``[b, Hq, S, D]``; k: ``[b, Hkv, S, D]``.  GQA (reading R10): query head
    ``h`` reads KV head ``h // (Hq // Hkv)``.  Reading R2: ``scale = 1/sqrt(D)``.
    """
    b, hq, S, D = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qp = pool_blocks(q, block)  # [b, Hq, NB, D]
    kp = pool_blocks(k, block)  # [b, Hkv, NB, D]
    nb = qp.shape[2]
    s = np.full((b, hq, nb, nb), -np.inf)
    for bi in range(b):
        for h in range(hq):
            full = scale * (qp[bi, h] @ kp[bi, h // G].T)  # [NB, NB]
            tri = np.tril(np.ones((nb, nb), dtype=bool))
            s[bi, h][tri] = full[tri]
    return s


def _head_param(budget: Mapping[str, Sequence[int]], key: str, h: int) -> int:
    return int(budget[key][h])


def select_blocks_prefill(q, k, budget: Mapping[str, Sequence[int]], block: int,
                          kmax: int | None = None, scale: float | None = None,
                          return_scores: bool = False):
    """Per-head top-k block selection for causal prefill.

    Row ``(b, h, m)`` has ``m + 1`` candidate key blocks (causal, reading R9),
    keeps ``budget_blocks(m + 1, ...)`` of them with the sink and the diagonal
    forced (reading R7: ``n_sink = n_local = 1`` in the configs), ranked by
    ``prefill_block_scores``.

    Returns ``block_idx[b, Hq, NB, kmax]`` (int32, ascending, padded with -1) and
    ``block_cnt[b, Hq, NB]`` (int32); with ``return_scores`` also the fp64
    scores.
    """
    s = prefill_block_scores(q, k, block, scale)
    b, hq, nb, _ = s.shape
    cnt = np.zeros((b, hq, nb), dtype=np.int32)
    sels = {}
    for bi in range(b):
        for h in range(hq):
            for m in range(nb):
                kk = budget_blocks(m + 1, _head_param(budget, "min_blocks", h),
                                   _head_param(budget, "ratio_q16", h))
                sel = select_row(s[bi, h, m, : m + 1], kk,
                                 _head_param(budget, "n_sink", h),
                                 _head_param(budget, "n_local", h))
                sels[bi, h, m] = sel
                cnt[bi, h, m] = len(sel)
    if kmax is None:
        kmax = int(cnt.max()) if cnt.size else 0
    idx = np.full((b, hq, nb, kmax), -1, dtype=np.int32)
    for (bi, h, m), sel in sels.items():
        if len(sel) > kmax:
            raise ValueError("kmax too small")
        idx[bi, h, m, : len(sel)] = sel
    if return_scores:
        return idx, cnt, s
    return idx, cnt


# ----------------------------------------------------------------------------
# O5  attention over the gathered blocks (S-HPLB summaries §1; Spin §2.A
#     "Attention"); O5' the same as a dense masked softmax
# ----------------------------------------------------------------------------


def _softmax_rows(z: np.ndarray, v: np.ndarray):
    """o = softmax(z) @ v and lse = log sum exp z, row by row, with the row
    maximum subtracted first.  Rows with no finite entry give o = 0, lse = -inf."""
    mu = np.max(z, axis=-1, keepdims=True)
    ok = np.isfinite(mu)
    mu_safe = np.where(ok, mu, 0.0)
    e = np.exp(z - mu_safe)
    den = e.sum(axis=-1, keepdims=True)
    o = np.where(ok, (e @ v) / np.where(den > 0, den, 1.0), 0.0)
    lse = np.where(ok[..., 0], mu_safe[..., 0] + np.log(np.where(den[..., 0] > 0, den[..., 0], 1.0)), -np.inf)
    return o, lse


def attention_prefill_gather(q, k, v, block_idx, block_cnt, block: int,
                             scale: float | None = None, tiles=None):
    """Causal attention of each query row over the keys of its tile's selected
    blocks only (block-gather form).

    Row ``t`` of query block ``m`` of head ``h`` attends to every key ``t' <= t``
    lying in a block listed in ``block_idx[b, h, m, :block_cnt[b, h, m]]`` of KV
    head ``h // G``.  ``tiles``: optional iterable of ``(b, h, m)`` to compute
    (the others stay NaN).  Returns ``o[b, Hq, S, D]`` and ``lse[b, Hq, S]``
    (natural log).
    """
    b, hq, S, D = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nb = -(-S // block)
    o = np.full((b, hq, S, D), np.nan)
    lse = np.full((b, hq, S), np.nan)
    if tiles is None:
        tiles = itertools.product(range(b), range(hq), range(nb))
    kcache: dict = {}
    for bi, h, m in tiles:
        j = h // G
        if (bi, j) not in kcache:
            kcache.clear()
            kcache[bi, j] = (to_f64(k[bi, j]), to_f64(v[bi, j]))
        kk, vv = kcache[bi, j]
        lo, hi = m * block, min(S, (m + 1) * block)
        qt = to_f64(q[bi, h, lo:hi])
        sel = [int(n) for n in block_idx[bi, h, m, : int(block_cnt[bi, h, m])]]
        keys = np.concatenate([np.arange(n * block, min(S, (n + 1) * block)) for n in sel]) if sel \
            else np.zeros(0, dtype=np.int64)
        z = scale * (qt @ kk[keys].T)
        rows = np.arange(lo, hi)[:, None]
        z = np.where(keys[None, :] <= rows, z, -np.inf)
        ot, lt = _softmax_rows(z, vv[keys])
        o[bi, h, lo:hi] = ot
        lse[bi, h, lo:hi] = lt
    return o, lse


def attention_prefill_dense_masked(q, k, v, block_idx, block_cnt, block: int,
                                   scale: float | None = None):
    """The same attention as a dense ``S x S`` masked softmax (form O5').

    ``M[t, t'] = 1`` iff block ``t' // block`` is selected for ``(h, t // block)``
    and ``t' <= t``; ``Z = scale * Q K^T`` with ``-inf`` where ``M = 0``;
    ``O = softmax(Z) V``.  Only for small shapes.
    """
    b, hq, S, D = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.empty((b, hq, S, D))
    lse = np.empty((b, hq, S))
    blk = np.arange(S) // block
    for bi in range(b):
        for h in range(hq):
            nb = block_idx.shape[2]
            selm = np.zeros((nb, nb), dtype=bool)
            for m in range(nb):
                for n in block_idx[bi, h, m, : int(block_cnt[bi, h, m])]:
                    selm[m, int(n)] = True
            mask = selm[blk[:, None], blk[None, :]] & (np.arange(S)[None, :] <= np.arange(S)[:, None])
            z = scale * (to_f64(q[bi, h]) @ to_f64(k[bi, h // G]).T)
            z = np.where(mask, z, -np.inf)
            o[bi, h], lse[bi, h] = _softmax_rows(z, to_f64(v[bi, h // G]))
    return o, lse


def prefill_tile_loads(block_cnt) -> np.ndarray:
    """LPT item loads for prefill (reading R21): item ``i = h * NB + m`` of
    sequence 0 has load ``k(h, m)``, the number of key blocks it attends to."""
    return np.asarray(block_cnt, dtype=np.int64).reshape(-1)


def attended_flops_prefill(block_idx, block_cnt, S: int, block: int, D: int) -> int:
    """Algorithmic flops of the attention: 4*D per visible (query, key) pair
    (2*D for Q K^T, 2*D for P V); the diagonal block counts its causal half."""
    b, hq, nb, _ = np.asarray(block_idx).shape
    pairs = 0
    for bi in range(b):
        for h in range(hq):
            for m in range(nb):
                rows = min(S, (m + 1) * block) - m * block
                for n in block_idx[bi, h, m, : int(block_cnt[bi, h, m])]:
                    n = int(n)
                    if n == m:
                        pairs += rows * (rows + 1) // 2
                    else:
                        pairs += rows * (min(S, (n + 1) * block) - n * block)
    return 4 * D * pairs


# ----------------------------------------------------------------------------
# decode: one query token per sequence at position L-1, per-head granularity
# (Fluxion summary, Intuizioni Chiave 2 and Componenti di Sistema)
# ----------------------------------------------------------------------------


def decode_select(q, k, budget: Mapping[str, Sequence[int]], kmax: int | None = None,
                  scale: float | None = None, return_scores: bool = False):
    """Per-head top-k block selection for one decode query per sequence.

    q: ``[b, Hq, D]``; k: ``[b, Hkv, L, D]``.  Head ``h`` uses its own block
    granularity ``g = budget['granularity'][h]``; its ``ceil(L / g)`` candidate
    blocks are scored against the mean-pooled keys of KV head ``h // G`` and the
    budget rule picks ``k`` of them (sink and local blocks forced).  A head whose
    budget equals its forced set (a streaming head, reading R7) needs no score.

    Returns ``block_idx[b, Hq, kmax]`` (ascending, -1 padded), ``block_cnt[b, Hq]``
    and, with ``return_scores``, a dict ``(b, h) -> fp64 scores``.
    """
    b, hq, D = q.shape
    hkv, L = k.shape[1], k.shape[2]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    sels, scores = {}, {}
    pooled: dict = {}
    for bi in range(b):
        pooled.clear()
        for h in range(hq):
            g = _head_param(budget, "granularity", h)
            j = h // G
            nc = -(-L // g)
            kk = budget_blocks(nc, _head_param(budget, "min_blocks", h), _head_param(budget, "ratio_q16", h))
            ns, nl = _head_param(budget, "n_sink", h), _head_param(budget, "n_local", h)
            if kk == len(forced_blocks(nc, ns, nl)):
                s = np.zeros(nc)  # ranking irrelevant: nothing beyond the forced set is kept
            else:
                if (j, g) not in pooled:
                    pooled[j, g] = pool_blocks(k[bi, j], g)
                s = scale * (pooled[j, g] @ to_f64(q[bi, h]))
            sels[bi, h] = select_row(s, kk, ns, nl)
            scores[bi, h] = s
    cnt = np.zeros((b, hq), dtype=np.int32)
    for key, sel in sels.items():
        cnt[key] = len(sel)
    if kmax is None:
        kmax = int(cnt.max())
    idx = np.full((b, hq, kmax), -1, dtype=np.int32)
    for (bi, h), sel in sels.items():
        if len(sel) > kmax:
            raise ValueError("kmax too small")
        idx[bi, h, : len(sel)] = sel
    if return_scores:
        return idx, cnt, scores
    return idx, cnt


def decode_attention(q, k, v, block_idx, block_cnt, granularity: Sequence[int],
                     scale: float | None = None, seqs=None):
    """Attention of each decode query (position ``L-1``, sees all ``L`` cached
    tokens, reading R9) over the tokens of its selected blocks only.

    Returns ``o[b, Hq, D]`` and ``lse[b, Hq]``; rows of sequences not in
    ``seqs`` stay NaN.
    """
    b, hq, D = q.shape
    hkv, L = k.shape[1], k.shape[2]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.full((b, hq, D), np.nan)
    lse = np.full((b, hq), np.nan)
    for bi in (range(b) if seqs is None else seqs):
        for h in range(hq):
            g = int(granularity[h])
            j = h // G
            sel = [int(n) for n in block_idx[bi, h, : int(block_cnt[bi, h])]]
            toks = np.concatenate([np.arange(n * g, min(L, (n + 1) * g)) for n in sel])
            kk = to_f64(k[bi, j, toks])
            z = scale * (kk @ to_f64(q[bi, h]))
            ot, lt = _softmax_rows(z[None, :], to_f64(v[bi, j, toks]))
            o[bi, h], lse[bi, h] = ot[0], lt[0]
    return o, lse


def decode_attention_dense(q, k, v, mask, scale: float | None = None):
    """Dense single-query attention with a token mask ``mask[b, Hq, L]`` (form
    O5' for decode)."""
    b, hq, D = q.shape
    hkv, L = k.shape[1], k.shape[2]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.empty((b, hq, D))
    lse = np.empty((b, hq))
    for bi in range(b):
        for h in range(hq):
            z = scale * (to_f64(k[bi, h // G]) @ to_f64(q[bi, h]))
            z = np.where(mask[bi, h], z, -np.inf)
            ot, lt = _softmax_rows(z[None, :], to_f64(v[bi, h // G]))
            o[bi, h], lse[bi, h] = ot[0], lt[0]
    return o, lse


# ----------------------------------------------------------------------------
# O6  greedy longest-load-first placement (S-HPLB summaries §2.B / §2.2)
# ----------------------------------------------------------------------------


def lpt_schedule(loads: Sequence[int], n_bins: int):
    """Greedy LPT: take the items by load, largest first (ties: lower item index
    first), and give each to the bin with the least load so far (ties: lower bin
    index).  Reading R22: a bin lists its items in the order they were assigned.

    Returns ``(bin_of_item[n] int32, bin_offsets[n_bins+1] int32,
    items_by_bin[n] int32, bin_load[n_bins] int64)``.
    """
    if n_bins <= 0:
        raise ValueError("n_bins must be positive")
    loads = [int(x) for x in loads]
    if any(x < 0 for x in loads):
        raise ValueError("loads must be non-negative")
    order = sorted(range(len(loads)), key=lambda i: (-loads[i], i))
    heap = [(0, bb) for bb in range(n_bins)]  # (load so far, bin)
    per_bin: list[list[int]] = [[] for _ in range(n_bins)]
    bin_of = np.empty(len(loads), dtype=np.int32)
    for i in order:
        cur, bb = heapq.heappop(heap)
        per_bin[bb].append(i)
        bin_of[i] = bb
        heapq.heappush(heap, (cur + loads[i], bb))
    bin_load = np.zeros(n_bins, dtype=np.int64)
    for cur, bb in heap:
        bin_load[bb] = cur
    offsets = np.zeros(n_bins + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(p) for p in per_bin])
    items = np.array([i for p in per_bin for i in p], dtype=np.int32)
    return bin_of, offsets, items, bin_load


def brute_force_makespan(loads: Sequence[int], n_bins: int) -> int:
    """Optimal makespan of multiway number partitioning by trying every
    assignment of items to bins (the NP-hard problem the S-HPLB summaries name
    in §2.B / §2.2).  Only for small instances (``n_bins ** n`` assignments)."""
    loads = np.asarray([int(x) for x in loads], dtype=np.int64)
    n = len(loads)
    if n == 0:
        return 0
    best = None
    # enumerate assignments in chunks of the first item fixed to bin 0 (symmetry)
    rest = n - 1
    digits = np.arange(n_bins ** rest, dtype=np.int64)
    assign = np.empty((digits.size, n), dtype=np.int64)
    assign[:, 0] = 0
    d = digits.copy()
    for i in range(1, n):
        assign[:, i] = d % n_bins
        d //= n_bins
    for bb in range(n_bins):
        part = ((assign == bb) * loads[None, :]).sum(axis=1)
        best = part if best is None else np.maximum(best, part)
    return int(best.min())
