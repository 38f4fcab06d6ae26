"""GPU parity of decode over a paged KV cache (per-KV-head page pools and a
page table, the page substrate of Spin's partitions).

The paged entry points compute with the same arithmetic in the same order as
the contiguous ones, so the pooled-key cache, the selected blocks and the
attention output must equal the contiguous path's bit for bit; and, on the
cache read back from the pages through the table, they meet the oracle under
the usual bars (block indices exact on pinned rows, 1e-2 max-abs for bf16).
"""

import numpy as np
import pytest
import torch

import oracle as O
from head_heterogeneous_block_amd import workloads as W

from gpu_helpers import check_row, max_abs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"
TOL_BF16 = 1e-2


def _say(*a):
    print(*a, flush=True)


def _pooled(plan):
    """The pooled-key cache the plan built (its buffer may be larger)."""
    return plan.k_pooled[:SA.sa_decode_pooled_size(plan.desc, plan.budgets) // 4]


def _run_both(inp, page_size, seed=7, out_f32=True):
    q, k, v = inp.q, inp.k, inp.v
    cont = SA.DecodePlan(q, k, v, inp.budget, out_f32=out_f32)
    oc = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=q.device)
    lc = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    cont.pool(k)
    cont.select(q, k)
    cont.attend(q, k, v, oc, lc)
    pk = W.make_paged(k, v, page_size, seed)
    paged = SA.PagedDecodePlan(q, pk.k_pages, pk.v_pages, pk.table, inp.spec.kv_len, inp.budget, out_f32=out_f32)
    op = torch.full_like(oc, float("nan"))
    lp = torch.full_like(lc, float("nan"))
    paged.pool(pk.k_pages)
    paged.select(q, pk.k_pages)
    paged.attend(q, pk.k_pages, pk.v_pages, op, lp)
    torch.cuda.synchronize()
    return cont, oc, lc, paged, op, lp, pk


def _gather_back(pk, b, hk, L):
    """Host copy of the cache read back from the pools through the page table."""
    kp, vp, tab = W.to_numpy(pk.k_pages), W.to_numpy(pk.v_pages), pk.table.cpu().numpy()
    D = kp.shape[-1]
    k = np.stack([np.stack([kp[j][tab[bi, j]].reshape(-1, D)[:L] for j in range(hk)]) for bi in range(b)])
    v = np.stack([np.stack([vp[j][tab[bi, j]].reshape(-1, D)[:L] for j in range(hk)]) for bi in range(b)])
    return k, v


@pytest.mark.parametrize("page_size,L", [(64, 8192 + 40), (128, 1000), (256, 8192), (128, 40)],
                         ids=["p64-ragged", "p128-short", "p256", "p128-tiny"])
def test_paged_decode_bitwise_and_oracle(page_size, L):
    spec = W.DECODE_128K.with_(batch=3, kv_len=L, tok_lo=16 if L < 64 else 256, tok_hi=64 if L < 64 else 2048,
                              stream_local=4 if L < 64 else 16)
    _say("case: paged decode page", page_size, "L", L)
    inp = W.make_decode(spec, 41, device=DEV)
    cont, oc, lc, paged, op, lp, pk = _run_both(inp, page_size)
    assert torch.equal(_pooled(paged), _pooled(cont)), "pooled keys differ"
    assert torch.equal(paged.block_idx, cont.block_idx) and torch.equal(paged.block_cnt, cont.block_cnt)
    assert torch.equal(op, oc) and torch.equal(lp, lc), "paged output differs from the contiguous path"
    # the oracle on the cache as the pages hold it
    k, v = _gather_back(pk, spec.batch, spec.n_kv_heads, L)
    q = W.to_numpy(inp.q)
    gidx, gcnt = paged.block_idx.cpu().numpy(), paged.block_cnt.cpu().numpy()
    oidx, ocnt, sc = O.decode_select(q, k, inp.budget, kmax=paged.kmax, return_scores=True)
    pinned = 0
    for bi in range(spec.batch):
        for h in range(spec.n_q_heads):
            g = int(inp.budget["granularity"][h])
            c = int(ocnt[bi, h])
            assert int(gcnt[bi, h]) == c
            F = O.forced_blocks(-(-L // g), int(inp.budget["n_sink"][h]), int(inp.budget["n_local"][h]))
            pinned += bool(check_row(gidx[bi, h, :c], oidx[bi, h, :c], sc[bi, h], c, F))
    ro, rl = O.decode_attention(q, k, v, gidx, gcnt, inp.budget["granularity"])
    err, lerr = max_abs(op.cpu().numpy(), ro), max_abs(lp.cpu().numpy(), rl)
    _say("pinned", pinned, "max abs err o", err, "lse", lerr)
    assert err <= TOL_BF16 and lerr <= TOL_BF16


@pytest.mark.parametrize("over", [dict(head_dim=64), dict(n_q_heads=16, n_kv_heads=2, n_streaming=4)],
                         ids=["d64", "gqa8"])
def test_paged_decode_other_shapes(over):
    """64-dim heads and eight query heads per KV head through pages: bitwise the
    contiguous path's pooled keys, selections and outputs (that path is checked
    against the oracle on the same shapes)."""
    spec = W.DECODE_128K.with_(batch=2, kv_len=4096 + 24, tok_lo=256, tok_hi=1024, stream_local=8, **over)
    _say("case: paged decode", over)
    inp = W.make_decode(spec, 53, device=DEV)
    cont, oc, lc, paged, op, lp, pk = _run_both(inp, 128)
    assert torch.equal(_pooled(paged), _pooled(cont))
    assert torch.equal(paged.block_idx, cont.block_idx) and torch.equal(paged.block_cnt, cont.block_cnt)
    assert torch.equal(op, oc) and torch.equal(lp, lc)


def test_paged_decode_bf16_output_and_table_out_of_range():
    """bf16 output equals the contiguous path's bit for bit; a page-table entry
    outside the pool reads as zero keys and values instead of faulting (the
    unchecked path: the host-side debug checks, which reject such a table, are
    switched off for it)."""
    spec = W.DECODE_128K.with_(batch=2, kv_len=4096, tok_lo=256, tok_hi=1024, stream_local=8)
    inp = W.make_decode(spec, 43, device=DEV)
    cont, oc, lc, paged, op, lp, pk = _run_both(inp, 128, out_f32=False)
    assert op.dtype == torch.bfloat16 and torch.equal(op, oc)
    bad = pk.table.clone()
    bad[1, 0, 5] = pk.k_pages.shape[1] + 7  # sequence 1, KV head 0, tokens 640..767
    plan = SA.PagedDecodePlan(inp.q, pk.k_pages, pk.v_pages, bad, spec.kv_len, inp.budget, out_f32=True)
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    was = SA.sa_set_debug_checks(False)
    try:
        plan.pool(pk.k_pages)
        plan.select(inp.q, pk.k_pages)
        plan.attend(inp.q, pk.k_pages, pk.v_pages, o)
        torch.cuda.synchronize()
    finally:
        SA.sa_set_debug_checks(was)
    assert torch.isfinite(o).all()
    kz, vz = inp.k.clone(), inp.v.clone()
    kz[1, 0, 640:768] = 0
    vz[1, 0, 640:768] = 0
    ref = SA.DecodePlan(inp.q, kz, vz, inp.budget, out_f32=True)
    oz = torch.empty_like(o)
    ref.pool(kz)
    ref.select(inp.q, kz)
    ref.attend(inp.q, kz, vz, oz)
    torch.cuda.synchronize()
    assert torch.equal(_pooled(plan), _pooled(ref)) and torch.equal(o, oz)


def test_paged_decode_full_size():
    """The 16 x 131072-token decode workload held in 128-token pages: the same
    selections and outputs as the contiguous cache, bit for bit."""
    spec = W.DECODE_128K
    _say("case: full decode config, paged")
    inp = W.make_decode(spec, W.seed_of(W.DECODE_128K), device=DEV)
    cont, oc, lc, paged, op, lp, pk = _run_both(inp, 128)
    assert torch.equal(_pooled(paged), _pooled(cont))
    assert torch.equal(paged.block_idx, cont.block_idx)
    assert torch.equal(op, oc) and torch.equal(lp, lc)
