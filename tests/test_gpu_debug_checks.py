"""The library's debug checks of the index tables (sa_set_debug_checks): with
them on, a valid call gives the same output as with them off, and a corrupt
block list, schedule, key-norm table or page table is rejected on the host with
SA_ERR_INVALID_ARG before anything is launched (the output buffer keeps its
fill)."""

import pytest
import torch

from head_heterogeneous_block_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"


@pytest.fixture
def checks_on():
    prev = SA.sa_set_debug_checks(True)
    yield
    SA.sa_set_debug_checks(prev)


def _rejected(fn, o, what):
    o.fill_(123.0)
    with pytest.raises(SA.SaError) as e:
        fn()
    assert e.value.status == SA.SA_ERR_INVALID_ARG and what in str(e.value), str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 123.0).all()), "a rejected call launched work"


def test_prefill_tables_checked(checks_on):
    spec = W.LLAMA_32K.with_(seq_len=4096, n_q_heads=8, n_kv_heads=2)
    print(f"debug checks prefill {spec}", flush=True)
    inp = W.make_prefill(spec, W.seed_of(W.LLAMA_32K), device=DEV)
    plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=64, out_f32=True, queue=True,
                          queues=8, queue_group="kv_tiers")
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    plan.select(inp.q, inp.k)
    SA.sa_set_debug_checks(False)
    plan.attend(inp.q, inp.k, inp.v, o)
    ref = o.clone()
    SA.sa_set_debug_checks(True)
    o.zero_()
    plan.attend(inp.q, inp.k, inp.v, o)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    good_idx, good_cnt, good_items = plan.block_idx.clone(), plan.block_cnt.clone(), plan.items_by_bin.clone()
    att = lambda: plan.attend(inp.q, inp.k, inp.v, o)  # noqa: E731
    # a block after the query block (causality) in row m = 5
    plan.block_idx[0, 1, 5, 0] = 6
    _rejected(att, o, "outside")
    plan.block_idx.copy_(good_idx)
    # a repeated block
    plan.block_idx[0, 2, 9, 1] = plan.block_idx[0, 2, 9, 0]
    _rejected(att, o, "strictly increasing")
    plan.block_idx.copy_(good_idx)
    # a count above kmax
    plan.block_cnt[0, 3, 7] = plan.kmax + 1
    _rejected(att, o, "block_cnt")
    plan.block_cnt.copy_(good_cnt)
    # a tile listed twice in the queue order
    plan.items_by_bin[1] = plan.items_by_bin[0]
    _rejected(att, o, "twice")
    plan.items_by_bin.copy_(good_items)
    # a key-norm entry below its block's longest key (the bound would be
    # wrong); one just above it passes
    good_norms = plan.key_norms.clone()
    plan.key_norms[0, 1, 17] *= 0.99
    _rejected(att, o, "key_norms[0][1][17]")
    plan.key_norms.copy_(good_norms)
    plan.key_norms[0, 0, 3] *= 1.01
    o.zero_()
    att()
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    plan.key_norms.copy_(good_norms)
    o.zero_()
    att()
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


def test_decode_tables_checked(checks_on):
    spec = W.DECODE_128K.with_(batch=2, kv_len=8192)
    print(f"debug checks decode {spec}", flush=True)
    inp = W.make_decode(spec, W.seed_of(W.DECODE_128K), device=DEV)
    pk = W.make_paged(inp.k, inp.v, 128, 5)
    plan = SA.PagedDecodePlan(inp.q, pk.k_pages, pk.v_pages, pk.table, spec.kv_len, inp.budget, out_f32=True)
    plan.pool(pk.k_pages)
    plan.select(inp.q, pk.k_pages)
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    att = lambda: plan.attend(inp.q, pk.k_pages, pk.v_pages, o)  # noqa: E731
    att()
    torch.cuda.synchronize()
    ref = o.clone()
    good_idx = plan.block_idx.clone()
    # head 20 is a retrieval head: its blocks lie in [0, ceil(L / granularity))
    g = int(inp.budget["granularity"][20])
    plan.block_idx[1, 20, 0] = -(-spec.kv_len // g)
    _rejected(att, o, "outside")
    plan.block_idx.copy_(good_idx)
    good_table = pk.table.clone()
    pk.table[1, 1, 3] = pk.k_pages.shape[1]  # one past the pool
    _rejected(att, o, "page table")
    pk.table.copy_(good_table)
    o.zero_()
    att()
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
