"""GPU parity of the prefill block selection (one kernel: query pooling, block
scores and top-k) on the shapes that change its layout: sequences long enough
that a workgroup holds fewer than 16 query-block rows in LDS (2048 blocks: 8
rows; 8192 blocks, the largest supported: 2 rows), a block count that leaves
the last workgroup ragged, and fp32 inputs.  Rows are checked under the parity rules of gpu_helpers.check_row
against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from head_heterogeneous_block_amd import workloads as W

from gpu_helpers import check_row

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _select(inp):
    spec = inp.spec
    plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block)
    plan.select(inp.q, inp.k)
    torch.cuda.synchronize()
    return plan, plan.block_idx.cpu().numpy(), plan.block_cnt.cpu().numpy()


def _check(inp, gidx, gcnt, rows=None):
    spec = inp.spec
    q, k = W.to_numpy(inp.q), W.to_numpy(inp.k)
    oidx, ocnt, sc = O.select_blocks_prefill(q, k, inp.budget, spec.block, kmax=gidx.shape[-1], return_scores=True)
    np.testing.assert_array_equal(gcnt, ocnt)
    nb = gcnt.shape[-1]
    kinds = [0, 0, 0]
    for bi in range(gcnt.shape[0]):
        for h in range(gcnt.shape[1]):
            for m in (range(nb) if rows is None else rows):
                c = int(ocnt[bi, h, m])
                assert np.all(gidx[bi, h, m, c:] == -1)
                F = O.forced_blocks(m + 1, int(inp.budget["n_sink"][h]), int(inp.budget["n_local"][h]))
                kinds[check_row(gidx[bi, h, m, :c], oidx[bi, h, m, :c], sc[bi, h, m, : m + 1], c, F)] += 1
    _say("rows exempt / gap-pinned / tie-pinned:", kinds)
    assert kinds[1] + kinds[2] >= 0.9 * sum(kinds)


@pytest.mark.parametrize("name,over", [
    ("2048-blocks", dict(seq_len=2048 * 64, n_q_heads=2, n_kv_heads=1, head_dim=64, block=64)),
    ("ragged-1000-blocks", dict(seq_len=999 * 64 + 13, n_q_heads=4, n_kv_heads=2, head_dim=128, block=64)),
    ("fp32-d128", dict(seq_len=300 * 64 + 5, n_q_heads=2, n_kv_heads=1, head_dim=128, block=64, dtype="f32")),
])
def test_select_layouts_all_rows(name, over):
    spec = W.LLAMA_32K.with_(**over)
    _say("case:", name, spec)
    inp = W.make_prefill(spec, 31, device=DEV)
    _, gidx, gcnt = _select(inp)
    _check(inp, gidx, gcnt)


def test_select_largest_block_count_sampled_rows():
    spec = W.LLAMA_32K.with_(seq_len=8192 * 64, n_q_heads=1, n_kv_heads=1, head_dim=64, block=64)
    _say("case: 8192 blocks", spec)
    inp = W.make_prefill(spec, 41, device=DEV)
    _, gidx, gcnt = _select(inp)
    rng = np.random.default_rng(41)
    rows = sorted(set(list(range(40)) + list(range(8192 - 40, 8192)) + rng.integers(0, 8192, 120).tolist()))
    _check(inp, gidx, gcnt, rows)

