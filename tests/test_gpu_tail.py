"""The prefill launch that records each workgroup's start and end
(sa_sparse_attn_prefill_timed): same output bits as the untimed launch, one
[start, end] pair per workgroup with start <= end, all inside the launch, for
every schedule and both prefill kernels."""

import pytest
import torch

from head_heterogeneous_block_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("sched", ["natural", "bins", "queue", "queue_xcd"])
def test_timed_prefill_stamps(sched, variant):
    spec = W.LLAMA_32K.with_(seq_len=4096 + 128, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, 90, device=DEV)
    kw = {"natural": dict(n_bins=0), "bins": dict(n_bins=37),
          "queue": dict(n_bins=23, queue=True, queues=1, queue_group="kv_tiers"),
          "queue_xcd": dict(n_bins=23, queue=True, queues=8, queue_group="kv_tiers")}[sched]
    plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, out_f32=True, kernel_variant=variant, **kw)
    plan.select(inp.q, inp.k)
    o1 = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    o2 = torch.empty_like(o1)
    plan.attend(inp.q, inp.k, inp.v, o1)
    t = plan.attend_timed(inp.q, inp.k, inp.v, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    t = t.cpu()
    assert t.shape == (plan.grid(), 2)
    assert bool((t[:, 0] > 0).all()) and bool((t[:, 1] >= t[:, 0]).all())
    span = int(t[:, 1].max() - t[:, 0].min())
    # the constant clock runs at about 100 MHz: a launch of these sizes spans
    # well under a second
    assert 0 < span < 100_000_000
