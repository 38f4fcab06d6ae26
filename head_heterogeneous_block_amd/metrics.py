"""Work accounting for the benchmark: algorithmic flops of the prefill attention
and algorithmic bytes of a decode step, from the selected block tables.

Pure bookkeeping over index tables (numpy); no attention arithmetic.
"""

from __future__ import annotations

import numpy as np

# MI355X published peaks (dense, no sparsity): bf16 MFMA and HBM3E bandwidth
PEAK_BF16_FLOPS = 2.5e15
PEAK_F32_MFMA_FLOPS = 157.3e12
PEAK_HBM_BYTES = 8.0e12


def prefill_pairs(block_idx: np.ndarray, block_cnt: np.ndarray, S: int, B: int) -> int:
    """Visible (query, key) pairs of a causal block-sparse prefill: a selected
    block below the diagonal contributes rows(m) * cols(n) pairs, the diagonal
    block rows(m) * (rows(m) + 1) / 2."""
    b, h, nb, kmax = block_idx.shape
    m = np.broadcast_to(np.arange(nb)[None, None, :, None], block_idx.shape)
    valid = np.arange(kmax)[None, None, None, :] < block_cnt[..., None]
    n = np.where(valid, block_idx, -1)
    rows = np.minimum(S, (m + 1) * B) - m * B
    cols = np.where(n >= 0, np.minimum(S, (n + 1) * B) - n * B, 0)
    pairs = np.where(n == m, rows * (rows + 1) // 2, rows * cols)
    pairs = np.where(valid, pairs, 0)
    return int(pairs.sum(dtype=np.int64))


def prefill_flops(block_idx, block_cnt, S: int, B: int, D: int) -> int:
    """4*D flops per visible pair: 2*D for Q K^T and 2*D for P V."""
    return 4 * D * prefill_pairs(block_idx, block_cnt, S, B)


def prefill_mfma_flops(block_cnt, B: int, D: int) -> int:
    """Flops the MFMA units issue: 64-key steps in full, except the steps of the
    diagonal block that lie wholly above the diagonal for a wave (skipped)."""
    return 4 * D * B * B * int(np.asarray(block_cnt, dtype=np.int64).sum())


def decode_bytes(block_idx: np.ndarray, block_cnt: np.ndarray, granularity, n_q_heads: int, n_kv_heads: int,
                 kv_len: int, head_dim: int, elem_bytes: int, scoring_heads) -> dict:
    """Algorithmic bytes of one decode step.

    kv: K and V rows of the union of the tokens the query heads of a KV group
        selected (read once per group); pooled: fp32 pooled keys scanned by the
        scoring heads (once per KV head and granularity); small: q, o, indices.
    """
    b = block_idx.shape[0]
    G = n_q_heads // n_kv_heads
    n_atoms = -(-kv_len // 16)
    union_tokens = 0
    for bi in range(b):
        for j in range(n_kv_heads):
            mark = np.zeros(n_atoms + 64, dtype=bool)
            for gi in range(G):
                h = j * G + gi
                g = int(granularity[h])
                sel = block_idx[bi, h, : int(block_cnt[bi, h])]
                apb = g // 16
                at = (sel[:, None] * apb + np.arange(apb)[None, :]).reshape(-1)
                mark[at[at < n_atoms]] = True
            atoms = np.flatnonzero(mark[:n_atoms])
            toks = np.minimum(kv_len, (atoms + 1) * 16) - atoms * 16
            union_tokens += int(toks.sum())
    kv = union_tokens * 2 * head_dim * elem_bytes
    pooled = 0
    for j in range(n_kv_heads):
        gs = sorted({int(granularity[h]) for h in range(j * G, (j + 1) * G) if scoring_heads[h]})
        for g in gs:
            pooled += b * (-(-kv_len // g)) * head_dim * 4
    small = b * n_q_heads * (2 * head_dim * elem_bytes + block_idx.shape[2] * 4 + 4)
    return {"kv": kv, "pooled": pooled, "small": small, "total": kv + pooled + small,
            "union_tokens": union_tokens}


def _lowbias32(x: np.ndarray) -> np.ndarray:
    """The "lowbias32" integer hash (C. Wellons, "Prospecting for Hash
    Functions") on uint32 arrays, wrapping like the GPU's 32-bit arithmetic."""
    x = x.astype(np.uint64)
    m = np.uint64(0xFFFFFFFF)
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(0x7FEB352D)) & m
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(0x846CA68B)) & m
    x ^= x >> np.uint64(16)
    return x


def mfma_probe_random_sink(n_workgroups: int, iters: int):
    """The sink of the MFMA rate probe with random operands (the header's
    formula, in fp64): per global thread, iters times the sum over the 8 chains
    of the accumulator entry each chain leaves in that lane's element c.
    Returns (expected, scale): scale is the same sum over the absolute products,
    against which the probe's fp32 accumulation error is measured."""
    import torch

    n = n_workgroups * 256
    t = np.arange(n, dtype=np.uint64)
    f = np.arange(8, dtype=np.uint64)
    e = np.arange(8, dtype=np.uint64)
    h = _lowbias32((64 * t[:, None, None] + 8 * f[None, :, None] + e[None, None, :]) & np.uint64(0xFFFFFFFF))
    v = ((h & np.uint64(0xFFFF)).astype(np.int64) - 32768).astype(np.float32) / np.float32(32768.0)
    v = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()  # round to nearest even
    w = v.reshape(n // 64, 64, 8, 8)  # wave, lane, fragment, element
    # fragment rows (A) / columns (B) are lane % 32; k = 8 * (lane / 32) + e
    frag = np.concatenate([w[:, :32], w[:, 32:]], axis=-1)  # wave, row, fragment, k (16)
    lane = np.arange(64)
    expected = np.zeros((n // 64, 64))
    scale = np.zeros((n // 64, 64))
    for c in range(8):
        a = frag[:, :, c % 4, :]          # wave, i, k
        b = frag[:, :, 4 + c % 4, :]      # wave, j, k
        d = np.einsum("wik,wjk->wij", a, b)
        dabs = np.einsum("wik,wjk->wij", np.abs(a), np.abs(b))
        row = 8 * (c // 4) + 4 * (lane // 32) + c % 4
        expected += d[:, row, lane % 32]
        scale += dabs[:, row, lane % 32]
    return (iters * expected).reshape(-1), (iters * scale).reshape(-1)
