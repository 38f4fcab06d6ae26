"""The key-norm bound of the prefill attention.  The selection writes, for each
key block, the largest Euclidean norm of its key rows (a by-product of the key
pooling); the attention uses |score| <= |q| * that norm to skip the per-step
row max wherever no score can rise more than 64 (log2 units) above the running
max.  Checked here:
  * the table against the fp64 norms of the rows, for bf16 D = 128 and 64 and
    fp32, with a ragged last block;
  * scores that rise steeply after a tile's first step (later key blocks
    scaled by 3, so P grows to about 2^10 without a raise on the skip path),
    with and without the table, against the oracle;
  * a block whose keys are so long that the bound is far from the scores, so
    the kernel falls back to the row max, against the oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from head_heterogeneous_block_amd import workloads as W

from gpu_helpers import max_abs, prefill_gpu, to_host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"
TOL_BF16 = 1e-2


def _say(*a):
    print(*a, flush=True)


def _row_norm_max(k: np.ndarray, block: int) -> np.ndarray:
    """[b][h][n]: the largest fp64 Euclidean norm of the rows of each key block."""
    b, h, s, d = k.shape
    nb = -(-s // block)
    pad = np.zeros((b, h, nb * block - s, d))
    rows = np.linalg.norm(np.concatenate([k.astype(np.float64), pad], axis=2), axis=-1)
    return rows.reshape(b, h, nb, block).max(axis=-1)


@pytest.mark.parametrize("spec", [
    W.LLAMA_32K.with_(seq_len=2048 + 77, n_q_heads=8, n_kv_heads=2),
    W.LLAMA_32K.with_(seq_len=1024 + 5, n_q_heads=4, n_kv_heads=2, head_dim=64),
    W.TINY_F32.with_(seq_len=1024 + 33),
], ids=["bf16-d128", "bf16-d64", "f32-d64"])
def test_key_norm_table(spec):
    _say("case: key-norm table", spec)
    inp = W.make_prefill(spec, 5, device=DEV)
    plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, key_norms=True)
    plan.select(inp.q, inp.k)
    torch.cuda.synchronize()
    got = plan.key_norms.cpu().numpy().astype(np.float64)
    want = _row_norm_max(O.to_f64(W.to_numpy(inp.k)), spec.block)
    assert got.shape == want.shape
    assert np.all(np.abs(got - want) <= 1e-5 * want)


def _steep(seed: int, factor: float):
    """A 2K layer whose key blocks from the third on are scaled by `factor`."""
    spec = W.LLAMA_32K.with_(seq_len=2048 + 64, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, seed, device=DEV)
    k = inp.k.float()
    k[:, :, 2 * spec.block:] *= factor
    inp.k = k.to(inp.k.dtype)
    return spec, inp


def test_steep_scores():
    """Key blocks from the third on scaled by 3: their scores exceed the first
    block's row max by about 10 log2 units while the bound still allows the
    skip, so with the table P reaches about 2^10 with no raise; without it the
    lazy rule raises the max at +8.  Both within tolerance of the oracle, and
    not bitwise equal (the two paths round P differently)."""
    spec, inp = _steep(17, 3.0)
    q, k, v = to_host(inp)
    outs = {}
    for key_norms in (True, False):
        _say("case: steep scores, key_norms", key_norms)
        idx, cnt, o, lse, _ = prefill_gpu(inp, n_bins=32, queue=True, key_norms=key_norms)
        ro, rl = O.attention_prefill_gather(q, k, v, idx.cpu().numpy(), cnt.cpu().numpy(), spec.block)
        err, lerr = max_abs(o.cpu().numpy(), ro), max_abs(lse.cpu().numpy(), rl)
        _say("steep: key_norms", key_norms, "max abs err o", err, "lse", lerr, "lse range", float(rl.min()),
             float(rl.max()))
        assert lerr <= 1e-4
        assert err <= TOL_BF16
        outs[key_norms] = o
    assert not torch.equal(outs[True], outs[False])


def test_long_keys_fall_back_to_the_row_max():
    spec = W.LLAMA_32K.with_(seq_len=2048 + 64, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, 23, device=DEV)
    k = inp.k.float()
    # one key row per head in block 3, 30 times as long as the others: the
    # bound (about 500 log2 units) then exceeds every running max by far more
    # than 64 and each tile that visits block 3 takes the row max at every
    # step, while the logits stay small enough (lse below about 200) for fp32
    # to hold lse to 1e-4
    k[:, :, 3 * spec.block + 5] *= 30.0
    inp.k = k.to(inp.k.dtype)
    _say("case: long keys")
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins=32, queue=True, key_norms=True)
    kn = plan.key_norms.cpu().numpy()
    assert np.all(kn[:, :, 3] > 10 * np.delete(kn, 3, axis=2).max(axis=2))
    q, kh, v = to_host(inp)
    ro, rl = O.attention_prefill_gather(q, kh, v, idx.cpu().numpy(), cnt.cpu().numpy(), spec.block)
    err, lerr = max_abs(o.cpu().numpy(), ro), max_abs(lse.cpu().numpy(), rl)
    _say("long keys: max abs err o", err, "lse", lerr, "lse range", float(rl.min()), float(rl.max()))
    assert lerr <= 1e-4
    assert err <= TOL_BF16
