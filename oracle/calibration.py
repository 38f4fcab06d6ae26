"""fp64 CPU oracle: offline calibration of per-head budgets, written from the pages.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Plain, slow statements
of the calibration that precedes the path: the attention mass every query block
puts on every key block, the share of that mass a head keeps at a budget, the
budget a head needs for a target share, and the max-min shifting of budget from
heads that need little to heads that need much under a fixed total.

Source: "S-HPLB: Efficient LLM Attention Serving via Sparsity-Aware Head
Parallelism Load Balance" -- Italian summary §2.A (offline profiling to the
budget that recovers a share of the attention weight, e.g. 90%; max-min budget
shifting) and Chinese summary §2.1 (relative sparsity is stable per head; all
heads start with equal budgets and budget moves iteratively from high-sparsity
heads to low-sparsity heads with the total unchanged).

The output-aware variant follows "Fluxion" (Italian summary, Intuizioni Chiave 1
and Componenti di Sistema): a budget judged by how far the head's attention
output moves from dense attention, not by the attention weight it keeps (the
sink blocks hold much weight and little value norm).

Readings where the pages are silent (kept with the design notes as R32-R35, R37):
  R32  the "attention weight" of a key block for a query block is the sum, over
       the query rows of the block, of their exact causal softmax probabilities
       on the block's keys;
  R33  a head's recovery at a budget ratio is the mean over (sequence, query
       block) of the mass its best selection keeps (the forced sink and local
       blocks plus the k - |F| heaviest others, ties to the lowest index, with k
       from the exact budget rule) divided by the row's total mass; kept and
       total mass are summed in ascending block order;
  R34  budgets live on a grid of ratios r = i * step (units of 2^-16), 1 <= i,
       r <= 2^16; the budget a head needs for a target recovery is the smallest
       grid ratio that reaches it;
  R35  shifting: every head starts at total / H; repeatedly the head with the
       lowest recovery (lowest index on ties) receives one step from the head
       whose recovery stays highest after giving it (lowest index on ties),
       while that donor would still stay strictly above the receiver; heads
       stay within [step, 2^16];
  R37  the output deviation of head h at a budget is the relative Frobenius
       distance sqrt(sum (o_sparse - o_dense)^2) / sqrt(sum o_dense^2) over all
       sequences, query rows and channels of that head, o_dense being causal
       attention over every key; the head's relative contribution (its share of
       the layer output after the output projection) needs the projection
       weights and is left out.

Parity status: output_deviation is pinned by the split of dense attention
into the selected and the dropped keys (o_dense - o_sparse = w_out * (o_out -
o_sparse), w_out the dropped keys' softmax weight, from two separate
softmaxes), by zero at the full budget and for constant values, and by a
hand-computed two-key case; block_attention_mass is pinned by its row-sum identity, the
uniform-attention closed form and the full-attention softmax of
``torch.nn.functional.scaled_dot_product_attention``; head_recovery by its
full-budget and forced-only values and by brute force over block subsets;
maxmin_shift by brute force over every allocation on small grids.
"""

from __future__ import annotations

import math
from typing import Mapping, Sequence

import numpy as np

from .block_sparse import attention_prefill_gather, budget_blocks, select_blocks_prefill, select_row, to_f64


def block_attention_mass(q, k, block: int, scale: float | None = None) -> np.ndarray:
    """W[b, h, m, n]: the causal softmax probability mass that the query rows of
    block m of head h put on the keys of block n (n <= m; zero above), in fp64.

    q ``[b, Hq, S, D]``, k ``[b, Hkv, S, D]``; query head h reads KV head
    h // (Hq / Hkv).  Each row's probabilities sum to one, so row m of W sums
    to the number of query rows in block m.
    """
    qf, kf = to_f64(q), to_f64(k)
    b, H, S, D = qf.shape
    G = H // kf.shape[1]
    c = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nb = -(-S // block)
    W = np.zeros((b, H, nb, nb))
    causal = np.tril(np.ones((S, S), dtype=bool))
    for bi in range(b):
        for h in range(H):
            z = c * (qf[bi, h] @ kf[bi, h // G].T)
            z = np.where(causal, z, -np.inf)
            z -= z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p /= p.sum(axis=1, keepdims=True)
            for m in range(nb):
                rows = p[m * block:(m + 1) * block]
                for n in range(m + 1):
                    W[bi, h, m, n] = rows[:, n * block:(n + 1) * block].sum()
    return W


def row_recovery(w_row: Sequence[float], k: int, n_sink: int, n_local: int) -> float:
    """Share of a row's mass kept by its best selection of k blocks (R33)."""
    w = [float(x) for x in w_row]
    sel = select_row(w, k, n_sink, n_local)  # forced blocks + heaviest others, ascending
    kept = 0.0
    for n in sel:
        kept += w[n]
    total = 0.0
    for x in w:
        total += x
    return kept / total if total > 0 else 1.0


def head_recovery(W_h, ratio_q16: int, min_blocks: int, n_sink: int, n_local: int) -> float:
    """Recovery of one head at a budget ratio: W_h ``[b, nb, nb]`` (R33)."""
    W_h = np.asarray(W_h, dtype=np.float64)
    b, nb, _ = W_h.shape
    acc = 0.0
    for bi in range(b):
        for m in range(nb):
            kk = budget_blocks(m + 1, min_blocks, ratio_q16)
            acc += row_recovery(W_h[bi, m, :m + 1], kk, n_sink, n_local)
    return acc / (b * nb)


def recovery_table(W, budget: Mapping[str, Sequence[int]], step_q16: int) -> np.ndarray:
    """rec[h, i] = recovery of head h at ratio (i + 1) * step (R34)."""
    W = np.asarray(W, dtype=np.float64)
    H = W.shape[1]
    n_grid = 65536 // step_q16
    rec = np.zeros((H, n_grid))
    for h in range(H):
        for i in range(n_grid):
            rec[h, i] = head_recovery(W[:, h], (i + 1) * step_q16, int(budget["min_blocks"][h]),
                                      int(budget["n_sink"][h]), int(budget["n_local"][h]))
    return rec


def needed_ratio(rec_h: Sequence[float], target: float, step_q16: int) -> int:
    """Smallest grid ratio whose recovery reaches ``target`` (R34)."""
    for i, r in enumerate(rec_h):
        if r >= target:
            return (i + 1) * step_q16
    return len(rec_h) * step_q16


def maxmin_shift(rec: np.ndarray, total_q16: int, step_q16: int) -> list[int]:
    """Max-min budget shifting on a recovery table ``rec[h, i]`` (R35).

    Every head starts at total / H (a whole number of steps); while the head with
    the lowest recovery can take a step and some other head can give one while
    staying strictly above it, the step moves.  Returns the ratios (units 2^-16).
    """
    H, n_grid = rec.shape
    per = total_q16 // H
    assert per * H == total_q16 and per % step_q16 == 0 and step_q16 <= per <= 65536
    idx = [per // step_q16 - 1] * H  # grid index of each head's ratio
    while True:
        # receiver: lowest current recovery that can still grow
        b = -1
        for h in range(H):
            if idx[h] + 1 < n_grid and (b < 0 or rec[h, idx[h]] < rec[b, idx[b]]):
                b = h
        if b < 0:
            break
        # donor: highest recovery after giving one step
        a = -1
        for h in range(H):
            if h != b and idx[h] >= 1 and (a < 0 or rec[h, idx[h] - 1] > rec[a, idx[a] - 1]):
                a = h
        if a < 0 or not rec[a, idx[a] - 1] > rec[b, idx[b]]:
            break
        idx[a] -= 1
        idx[b] += 1
    return [(i + 1) * step_q16 for i in idx]


def brute_force_maxmin(rec: np.ndarray, total_q16: int, step_q16: int) -> float:
    """The largest achievable minimum recovery over every allocation of the
    total on the grid (heads within [step, 2^16]); small cases only."""
    H, n_grid = rec.shape
    units = total_q16 // step_q16
    best = -1.0

    def rec_min(alloc):
        return min(rec[h, alloc[h] - 1] for h in range(H))

    def walk(h, left, alloc):
        nonlocal best
        if h == H - 1:
            if 1 <= left <= n_grid:
                best = max(best, rec_min(alloc + [left]))
            return
        for u in range(1, min(n_grid, left - (H - 1 - h)) + 1):
            walk(h + 1, left - u, alloc + [u])

    walk(0, units, [])
    return best


def output_deviation(o_sparse, o_dense) -> np.ndarray:
    """dev[h] = ||o_sparse[:, h] - o_dense[:, h]||_F / ||o_dense[:, h]||_F over
    every sequence, row and channel of head h (R37); arrays ``[b, Hq, S, D]``."""
    a, r = to_f64(o_sparse), to_f64(o_dense)
    H = a.shape[1]
    dev = np.zeros(H)
    for h in range(H):
        num = 0.0
        den = 0.0
        for bi in range(a.shape[0]):
            d = a[bi, h] - r[bi, h]
            num += float(np.sum(d * d))
            den += float(np.sum(r[bi, h] * r[bi, h]))
        dev[h] = math.sqrt(num) / math.sqrt(den) if den > 0 else 0.0
    return dev


def deviation_table(q, k, v, budget: Mapping[str, Sequence[int]], block: int, step_q16: int) -> np.ndarray:
    """dev[h, i]: output deviation of head h when every head runs at ratio
    (i + 1) * step (R34, R37), the blocks chosen by the path's own selection
    (pooled scores, per-head top-k with the sink and local blocks), against
    causal attention over every key (ratio 1 keeps every block)."""
    n_grid = 65536 // step_q16
    H = q.shape[1]
    full = dict(budget)
    full["ratio_q16"] = [65536] * H
    idx, cnt = select_blocks_prefill(q, k, full, block)
    o_dense, _ = attention_prefill_gather(q, k, v, idx, cnt, block)
    dev = np.zeros((H, n_grid))
    for i in range(n_grid):
        b = dict(budget)
        b["ratio_q16"] = [(i + 1) * step_q16] * H
        idx, cnt = select_blocks_prefill(q, k, b, block)
        o, _ = attention_prefill_gather(q, k, v, idx, cnt, block)
        dev[:, i] = output_deviation(o, o_dense)
    return dev


def needed_ratio_deviation(dev_h: Sequence[float], max_dev: float, step_q16: int) -> int:
    """Smallest grid ratio whose output deviation is at most ``max_dev`` (R37)."""
    for i, d in enumerate(dev_h):
        if d <= max_dev:
            return (i + 1) * step_q16
    return len(dev_h) * step_q16

