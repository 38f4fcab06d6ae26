"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI
binding and compare it with the oracle under the parity rules.

Selection parity (block indices): a row is *pinned* when the oracle's fp64
score gap between the last kept and the best dropped non-forced block exceeds
1e-4 relative; pinned rows must match the oracle exactly.  Other rows (near
ties) must still hold the forced blocks, have the right count, and keep only
blocks whose score is within 1e-4 (relative) of the best dropped one.

Attention parity: the oracle attends over the GPU's own block lists, so the
attention check measures the attention kernel alone; the selection check covers
the lists themselves.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
from head_heterogeneous_block_amd import workloads as W

GAP = 1e-4


def gap_scale(a: float, b: float, row_max: float) -> float:
    return max(abs(a), abs(b), 1e-3 * row_max)


def check_row(gpu_sel, ora_sel, scores, k, forced):
    """Checks one selected row.  Returns 1 if the row was pinned by its score gap
    (exact match required), 2 if pinned by an exact tie (exact match required:
    ties go to the lowest block index), 0 if exempt (near tie: validity only).

    An exact tie is a row whose last kept and best dropped candidates have equal
    fp64 oracle scores (-0 and +0 compare equal), with every other candidate more
    than the gap away from that value, so the choice inside the tied set is
    decided by the tie rule alone."""
    gpu_sel = [int(x) for x in gpu_sel]
    ora_sel = [int(x) for x in ora_sel]
    assert len(gpu_sel) == k, (len(gpu_sel), k)
    assert gpu_sel == sorted(set(gpu_sel)), gpu_sel
    fs = set(forced)
    cand = [n for n in range(len(scores)) if n not in fs]
    kept = [n for n in ora_sel if n not in fs]
    dropped = [n for n in cand if n not in set(ora_sel)]
    if not kept or not dropped:
        assert gpu_sel == ora_sel
        return 1
    row_max = float(np.max(np.abs(scores[cand])))
    last_kept = min(scores[n] for n in kept)
    best_drop = max(scores[n] for n in dropped)
    scale = gap_scale(last_kept, best_drop, row_max)
    if last_kept - best_drop > GAP * scale:
        assert gpu_sel == ora_sel, (gpu_sel, ora_sel)
        return 1
    if last_kept == best_drop:
        others = [scores[n] for n in cand if scores[n] != last_kept]
        if all(abs(x - last_kept) > GAP * scale for x in others):
            assert gpu_sel == ora_sel, ("exact tie", gpu_sel, ora_sel)
            return 2
    assert fs <= set(gpu_sel)
    gkept = [n for n in gpu_sel if n not in fs]
    gdrop = [n for n in cand if n not in set(gpu_sel)]
    if gkept and gdrop:
        assert min(scores[n] for n in gkept) >= max(scores[n] for n in gdrop) - GAP * scale
    return 0


def check_prefill_selection(gpu_idx, gpu_cnt, ora_idx, ora_cnt, scores, budget, heads=None):
    """Compare [b, H, NB, kmax] tables; ``heads`` maps local head -> budget head."""
    b, H, nb = gpu_cnt.shape
    kinds = count_rows_prefill(gpu_idx, gpu_cnt, ora_idx, ora_cnt, scores, budget, heads)
    return kinds[1] + kinds[2], kinds[0]


def count_rows_prefill(gpu_idx, gpu_cnt, ora_idx, ora_cnt, scores, budget, heads=None):
    """check_row over every row; returns counts of [exempt, gap-pinned, tie-pinned]."""
    b, H, nb = gpu_cnt.shape
    kinds = [0, 0, 0]
    np.testing.assert_array_equal(gpu_cnt, ora_cnt)
    for bi in range(b):
        for h in range(H):
            hb = h if heads is None else heads[h]
            for m in range(nb):
                c = int(ora_cnt[bi, h, m])
                assert np.all(gpu_idx[bi, h, m, c:] == -1)
                F = O.forced_blocks(m + 1, int(budget["n_sink"][hb]), int(budget["n_local"][hb]))
                kinds[check_row(gpu_idx[bi, h, m, :c], ora_idx[bi, h, m, :c], scores[bi, h, m, : m + 1], c, F)] += 1
    return kinds


def prefill_gpu(inp: W.PrefillInputs, n_bins: int = 0, out_f32: bool = True, with_lse: bool = True,
                queue: bool = False, queues: int = 8, kernel_variant: int = 0, key_norms: bool = True,
                queue_group: str = "auto"):
    """Select + attend on the GPU; returns (block_idx, block_cnt, o, lse, plan) on the device."""
    from head_heterogeneous_block_amd import sparse_attn as SA
    q, k, v = inp.q, inp.k, inp.v
    plan = SA.PrefillPlan(q, k, v, inp.budget, inp.spec.block, n_bins=n_bins, out_f32=out_f32, queue=queue,
                          queues=queues, kernel_variant=kernel_variant, key_norms=key_norms, queue_group=queue_group)
    o = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if with_lse else None
    plan.select(q, k)
    plan.attend(q, k, v, o, lse)
    torch.cuda.synchronize()
    return plan.block_idx, plan.block_cnt, o, lse, plan


def to_host(inp):
    return W.to_numpy(inp.q), W.to_numpy(inp.k), W.to_numpy(inp.v)


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.isfinite(a)), "non-finite output"
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def bf16_half_ulp(x):
    """Half a unit in the last place of bf16 at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 1e-30)
    return np.exp2(np.floor(np.log2(ax)) - 8)
