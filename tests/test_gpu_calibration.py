"""GPU parity of the block attention mass (calibration input) against the fp64
oracle, and the calibration run end to end on it.

The mass sums exact softmax probabilities in fp32: each probability carries
about 1e-6 relative error, so a block pair's mass (at most 128 * 128
probabilities, summing to at most 128) is held to 2e-3 absolute; each row of
blocks must sum to its query-row count within the same bound.
"""

import numpy as np
import pytest
import torch

import oracle as O
from head_heterogeneous_block_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"
TOL_MASS = 2e-3


def _say(*a):
    print(*a, flush=True)


def _mass_gpu(inp):
    spec = inp.spec
    d = SA.make_prefill_desc(inp.q, inp.k, inp.v, inp.q, 128)
    nb = -(-spec.seq_len // 128)
    mass = torch.full((spec.batch, spec.n_q_heads, nb, nb), float("nan"), dtype=torch.float32, device=DEV)
    SA.sa_block_attention_mass(d, inp.q, inp.k, mass)
    torch.cuda.synchronize()
    return mass.cpu().numpy()


@pytest.mark.parametrize("name,over", [
    ("llama-2k", dict(seq_len=2048, n_q_heads=8, n_kv_heads=2)),
    ("ragged", dict(seq_len=1000, n_q_heads=4, n_kv_heads=2)),
    ("d64", dict(seq_len=1536, n_q_heads=4, n_kv_heads=1, head_dim=64)),
    ("one-block", dict(seq_len=100, n_q_heads=2, n_kv_heads=1)),
], ids=["llama-2k", "ragged", "d64", "one-block"])
def test_block_mass_against_oracle(name, over):
    spec = W.LLAMA_32K.with_(**over)
    _say("case: block mass", name)
    inp = W.make_prefill(spec, 51, device=DEV)
    got = _mass_gpu(inp)
    want = O.block_attention_mass(W.to_numpy(inp.q), W.to_numpy(inp.k), 128)
    err = float(np.max(np.abs(got - want)))
    _say("max abs err", err)
    assert np.all(np.isfinite(got)) and err <= TOL_MASS
    nb = got.shape[-1]
    rows = np.array([min(128, spec.seq_len - 128 * m) for m in range(nb)], dtype=np.float64)
    assert np.max(np.abs(got.sum(axis=3) - rows)) <= TOL_MASS
    assert np.all(np.triu(got, 1) == 0)


def test_calibration_end_to_end():
    """Mass on the GPU, recovery table and max-min shifting on the host: the
    shifted budgets keep a lowest-head recovery within 1e-3 of what the oracle's
    own mass and shifting reach, at the same total."""
    spec = W.LLAMA_32K.with_(seq_len=4096, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, 52, device=DEV)
    got = _mass_gpu(inp)
    want = O.block_attention_mass(W.to_numpy(inp.q), W.to_numpy(inp.k), 128)
    bud = {"min_blocks": [2] * 8, "ratio_q16": [0] * 8, "n_sink": [1] * 8, "n_local": [1] * 8}
    step = 2048
    total = 8 * 4096  # a mean budget of 1/16 of the causal blocks
    rec_g = SA.sa_budget_recovery(got, bud, step)
    rec_o = O.recovery_table(want, bud, step)
    assert np.max(np.abs(rec_g - rec_o)) <= 1e-3
    r_g = SA.sa_budget_shift(rec_g, step, total)
    r_o = O.maxmin_shift(rec_o, total, step)
    assert int(r_g.sum()) == total
    min_g = min(rec_o[h, r_g[h] // step - 1] for h in range(8))
    min_o = min(rec_o[h, r_o[h] // step - 1] for h in range(8))
    _say("lowest recovery: gpu-mass budgets", min_g, "oracle", min_o, "equal split", rec_o[:, total // 8 // step - 1].min())
    assert abs(min_g - min_o) <= 1e-3
    assert min_g >= rec_o[:, total // 8 // step - 1].min() - 1e-3


# ---------------------------------------------------------------- output deviation (output-aware criterion)


def test_output_deviation_kernel_and_table():
    """sa_output_deviation against the same sums in fp64 on the host (on the
    GPU's own arrays: only the summation order differs, so 1e-12 relative);
    deviation_table equal to a loop of the same calls; and, per ratio, the
    oracle's deviation on the GPU's selections (its attention over the same
    blocks) within the bound the attention error allows: with e_s, e_r the
    max-abs errors of the sparse and dense outputs over N elements,
    |dev' - dev| <= sqrt(N) (e_s + e_r (1 + dev)) / (||o_ref|| - sqrt(N) e_r)."""
    spec = W.LLAMA_32K.with_(batch=2, seq_len=1024 + 96, n_q_heads=4, n_kv_heads=2)
    _say("case: output deviation", spec.seq_len)
    inp = W.make_prefill(spec, 31, device=DEV)
    H, step = spec.n_q_heads, 16384
    q, k, v = W.to_numpy(inp.q), W.to_numpy(inp.k), W.to_numpy(inp.v)

    def run(ratio):
        b = dict(inp.budget)
        b["ratio_q16"] = [ratio] * H
        plan = SA.PrefillPlan(inp.q, inp.k, inp.v, b, spec.block, n_bins=64, out_f32=True, queue=True)
        o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
        plan.select(inp.q, inp.k)
        plan.attend(inp.q, inp.k, inp.v, o)
        return plan, o

    ref_plan, o_ref = run(65536)
    rho, _ = O.attention_prefill_gather(q, k, v, ref_plan.block_idx.cpu().numpy(), ref_plan.block_cnt.cpu().numpy(),
                                        spec.block)
    r_gpu = o_ref.cpu().numpy().astype(np.float64)
    e_r = float(np.max(np.abs(r_gpu - rho)))
    assert e_r <= 1e-2
    got = []
    for i in range(65536 // step):
        plan, o = run((i + 1) * step)
        dev = torch.full((H,), float("nan"), dtype=torch.float64, device=DEV)
        SA.sa_output_deviation(plan.desc, o, o_ref, dev)
        torch.cuda.synchronize()
        d_gpu = dev.cpu().numpy()
        got.append(d_gpu)
        a_gpu = o.cpu().numpy().astype(np.float64)
        host = np.array([np.sqrt(np.sum((a_gpu[:, h] - r_gpu[:, h]) ** 2)) / np.sqrt(np.sum(r_gpu[:, h] ** 2))
                         for h in range(H)])
        np.testing.assert_allclose(d_gpu, host, rtol=1e-12, atol=0)
        oo, _ = O.attention_prefill_gather(q, k, v, plan.block_idx.cpu().numpy(), plan.block_cnt.cpu().numpy(),
                                           spec.block)
        want = O.output_deviation(oo, rho)
        e_s = float(np.max(np.abs(a_gpu - oo)))
        assert e_s <= 1e-2
        n = a_gpu[:, 0].size
        bound = np.array([np.sqrt(n) * (e_s + e_r * (1 + want[h])) /
                          (np.sqrt(np.sum(rho[:, h] ** 2)) - np.sqrt(n) * e_r) for h in range(H)])
        _say("ratio", (i + 1) * step, "dev", d_gpu, "oracle", want, "bound", bound)
        assert np.all(np.abs(d_gpu - want) <= bound)
    assert np.all(np.stack(got)[-1] == 0.0)  # ratio 1 against itself
    table = SA.deviation_table(inp.q, inp.k, inp.v, inp.budget, spec.block, step, n_bins=64)
    np.testing.assert_array_equal(table, np.stack(got).T)
