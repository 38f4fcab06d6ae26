"""The binding's checks of tensor layouts against the descriptor (no GPU needed).

The kernels address every tensor from the descriptor's sizes and strides
alone, so a tensor of another shape, dtype or layout would be read or written
outside its storage.  The plans reject such calls with ValueError before the
library is called; a call that passes the checks reaches the library, which
returns SA_ERR_NO_DEVICE on a machine without a GPU.
"""

import pytest
import torch

from head_heterogeneous_block_amd import workloads as W

SA = pytest.importorskip("head_heterogeneous_block_amd.sparse_attn", reason="library not built", exc_type=ImportError)

pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="checks the host path on a machine without a GPU")


def _reaches_library(fn):
    with pytest.raises(SA.SaError) as e:
        fn()
    assert e.value.status == SA.SA_ERR_NO_DEVICE


def _prefill():
    spec = W.LLAMA_32K.with_(batch=2, seq_len=300, n_q_heads=4, n_kv_heads=2)
    inp = W.make_prefill(spec, 3)
    plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=8, out_f32=True, queue=True,
                          queues=2, queue_group="kv_tiers")
    return spec, inp, plan


def test_prefill_output_checks():
    spec, inp, plan = _prefill()
    q, k, v = inp.q, inp.k, inp.v
    o = torch.empty(q.shape, dtype=torch.float32)
    _reaches_library(lambda: plan.attend(q, k, v, o))
    # o laid out differently from q (token-major): accepted, its strides are used
    o_tm = torch.empty((q.shape[0], q.shape[2], q.shape[1], q.shape[3]), dtype=torch.float32).transpose(1, 2)
    _reaches_library(lambda: plan.attend(q, k, v, o_tm))
    assert list(plan.desc.o_stride) == list(o_tm.stride()[:3])
    with pytest.raises(ValueError, match="dtype"):  # a bf16 output for a plan that writes fp32
        plan.attend(q, k, v, torch.empty(q.shape, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        plan.attend(q, k, v, torch.empty((2, 4, 256, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="lse"):
        plan.attend(q, k, v, o, torch.empty((2, 4, 299), dtype=torch.float32))
    with pytest.raises(ValueError, match="lse"):
        plan.attend(q, k, v, o, torch.empty((2, 4, 300), dtype=torch.float64))
    with pytest.raises(ValueError, match="o must be"):
        plan.attend(q, k, v, o[0])


def test_prefill_input_checks():
    spec, inp, plan = _prefill()
    q, k, v = inp.q, inp.k, inp.v
    o = torch.empty(q.shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="k: shape"):
        plan.attend(q, k[:, :1], v, o)
    with pytest.raises(ValueError, match="v: dtype"):
        plan.attend(q, k, v.float(), o)
    # q of the right shape but another layout than the plan was built for
    q_tm = q.transpose(1, 2).contiguous().transpose(1, 2)
    with pytest.raises(ValueError, match="q: strides"):
        plan.select(q_tm, k)
    _reaches_library(lambda: plan.select(q, k))


def test_select_output_checks():
    spec, inp, plan = _prefill()
    args = (plan.desc, plan.budgets, inp.q, inp.k, None)
    with pytest.raises(ValueError, match="block_idx"):
        SA.sa_select_blocks(*args, plan.block_idx[..., :-1], plan.block_cnt, plan.kmax, plan.select_ws)
    with pytest.raises(ValueError, match="block_cnt"):
        SA.sa_select_blocks(*args, plan.block_idx, plan.block_cnt.long(), plan.kmax, plan.select_ws)
    with pytest.raises(ValueError, match="key_norms"):
        SA.sa_select_blocks(*args, plan.block_idx, plan.block_cnt, plan.kmax, plan.select_ws,
                            torch.empty((2, 2, 2), dtype=torch.float32))


def test_decode_checks():
    spec = W.DECODE_128K.with_(batch=2, kv_len=1000, tok_lo=64, tok_hi=256, stream_local=4)
    inp = W.make_decode(spec, 5)
    plan = SA.DecodePlan(inp.q, inp.k, inp.v, inp.budget, out_f32=True)
    q, k, v = inp.q, inp.k, inp.v
    o = torch.empty(q.shape, dtype=torch.float32)
    _reaches_library(lambda: plan.attend(q, k, v, o))
    with pytest.raises(ValueError, match="o: dtype"):
        plan.attend(q, k, v, torch.empty(q.shape, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse"):
        plan.attend(q, k, v, o, torch.empty((2, 31), dtype=torch.float32))
    with pytest.raises(ValueError, match="k: shape"):
        plan.attend(q, k[:, :, :999], v, o)
    with pytest.raises(ValueError, match="k: shape"):
        plan.pool(k[:1])
