"""The path captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed: the prefill selection and attention on the partitioned work queue,
the decode step, and the decode step through the allocation-free entry point.
Each graph is replayed several times with the program's own eager work and
synchronisations between the replays, and every replay must equal the eager
result bit for bit.  The library records no memset and no allocation: the
queue counters are cleared by a kernel, the decode plan rewrites its lists."""

import pytest
import torch

from head_heterogeneous_block_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"
REPLAYS = 3


def _say(*a):
    print(*a, flush=True)


def _capture(fn):
    """Warm fn up on a side stream (default priority), then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_prefill_graph_replays():
    spec = W.LLAMA_32K.with_(seq_len=4096 + 77, n_q_heads=8, n_kv_heads=2)
    _say("graph prefill", spec)
    inp = W.make_prefill(spec, 11, device=DEV)
    plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=64, out_f32=True, queue=True,
                          queues=8, queue_group="kv_tiers")
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(inp.q.shape[:3], dtype=torch.float32, device=DEV)
    step = lambda: (plan.select(inp.q, inp.k), plan.attend(inp.q, inp.k, inp.v, o, lse))  # noqa: E731
    step()
    torch.cuda.synchronize()
    ref = (plan.block_idx.clone(), plan.block_cnt.clone(), o.clone(), lse.clone())
    g = _capture(step)
    o2 = torch.empty_like(o)
    for r in range(REPLAYS):
        plan.block_idx.fill_(-7)
        plan.block_cnt.fill_(-7)
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (plan.block_idx, plan.block_cnt, o, lse)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {r} differs"
        # eager work of the program between the replays
        plan.attend(inp.q, inp.k, inp.v, o2)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref[2])


def test_graph_capture_with_debug_checks():
    """With the host-side checks on, the warm-up calls are checked and the
    captured calls skip them (a capture allows no synchronisation): the capture
    succeeds and every replay equals the eager result."""
    spec = W.LLAMA_32K.with_(seq_len=2048 + 5, n_q_heads=4, n_kv_heads=1)
    _say("graph prefill with debug checks", spec)
    inp = W.make_prefill(spec, 5, device=DEV)
    plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=32, out_f32=True, queue=True,
                          queues=2, queue_group="kv_tiers")
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    step = lambda: (plan.select(inp.q, inp.k), plan.attend(inp.q, inp.k, inp.v, o))  # noqa: E731
    was = SA.sa_set_debug_checks(True)
    try:
        step()
        torch.cuda.synchronize()
        ref = (plan.block_idx.clone(), plan.block_cnt.clone(), o.clone())
        g = _capture(step)
        for r in range(REPLAYS):
            o.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert all(torch.equal(a, b) for a, b in zip((plan.block_idx, plan.block_cnt, o), ref)), f"replay {r}"
    finally:
        SA.sa_set_debug_checks(was)


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_decode_graph_replays(noalloc):
    spec = W.DECODE_128K.with_(batch=3, kv_len=8192 + 40)
    _say("graph decode", spec, "noalloc" if noalloc else "workspace")
    inp = W.make_decode(spec, W.seed_of(W.DECODE_128K), device=DEV)
    plan = SA.DecodePlan(inp.q, inp.k, inp.v, inp.budget, out_f32=True)
    plan.pool(inp.k)
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device=DEV)

    def attend():
        if noalloc:
            SA.sa_sparse_attn_decode_noalloc(plan.desc, plan.budgets, inp.q, inp.k, inp.v, o, lse, plan.block_idx,
                                             plan.block_cnt, plan.kmax, out_f32=True)
        else:
            plan.attend(inp.q, inp.k, inp.v, o, lse)

    step = lambda: (plan.select(inp.q, inp.k), attend())  # noqa: E731
    step()
    torch.cuda.synchronize()
    ref = (plan.block_idx.clone(), plan.block_cnt.clone(), o.clone(), lse.clone())
    g = _capture(step)
    for r in range(REPLAYS):
        plan.block_idx.fill_(-7)
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (plan.block_idx, plan.block_cnt, o, lse)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {r} differs"
        step()  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(o, ref[2])
