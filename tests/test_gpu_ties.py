"""GPU selection under exact score ties: ties go to the lowest block index.

Gaussian inputs almost never tie, so these cases build ties on purpose, exact
in fp32 on the GPU and in fp64 in the oracle alike:

- Q = 0 (prefill) or q = 0 (decode): every block score is zero;
- every key block a copy of the first: every pooled key, hence every score of a
  row, is identical;
- key blocks duplicated in pairs: scores tie in pairs, so the selection boundary
  often falls inside a tied pair;
- decode q and keys on disjoint halves of the head dimension: every product in
  a score is a signed zero, so every score is zero.

Rows whose boundary is an exact tie (with every other score more than the 1e-4
gap away) must equal the oracle's selection element by element (both top-k
modes of the kernel: prefill rows and decode rows).  The attention over the
selected blocks is checked too.
"""

import numpy as np
import pytest
import torch

import oracle as O
from head_heterogeneous_block_amd import workloads as W

from gpu_helpers import check_row, count_rows_prefill, max_abs, prefill_gpu, to_host

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"
TOL_BF16 = 1e-2


def _say(*a):
    print(*a, flush=True)


def _prefill_case(inp):
    spec = inp.spec
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins=32, queue=True)
    q, k, v = to_host(inp)
    oidx, ocnt, scores = O.select_blocks_prefill(q, k, inp.budget, spec.block, kmax=plan.kmax, return_scores=True)
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    kinds = count_rows_prefill(gidx, gcnt, oidx, ocnt, scores, inp.budget)
    ro, rl = O.attention_prefill_gather(q, k, v, gidx, gcnt, spec.block)
    err = max_abs(o.cpu().numpy(), ro)
    _say("rows exempt / gap-pinned / tie-pinned", kinds, "max abs err o", err)
    assert err <= TOL_BF16
    return kinds


def _prefill_inputs(seed):
    spec = W.LLAMA_32K.with_(seq_len=4096, n_q_heads=8, n_kv_heads=2)
    return W.make_prefill(spec, seed, device=DEV)


def test_prefill_ties_zero_query():
    """Q = 0: every score is zero; each row keeps the sink, the diagonal and the
    lowest-index candidates."""
    inp = _prefill_inputs(81)
    inp.q = torch.zeros_like(inp.q)
    _say("case: prefill ties, Q = 0")
    kinds = _prefill_case(inp)
    assert kinds[0] == 0
    assert kinds[2] > 0


def test_prefill_ties_repeated_key_block():
    """Every key block a copy of block 0: all pooled keys are identical, so all
    scores of a row tie exactly."""
    inp = _prefill_inputs(82)
    B, S = inp.spec.block, inp.spec.seq_len
    inp.k = inp.k[:, :, :B].repeat(1, 1, S // B, 1).contiguous()
    _say("case: prefill ties, repeated key block")
    kinds = _prefill_case(inp)
    assert kinds[0] == 0
    assert kinds[2] > 0


def test_prefill_ties_paired_key_blocks():
    """Key block 2i+1 a copy of block 2i: scores tie in pairs, and rows whose
    budget boundary falls inside a pair must keep its lower block."""
    inp = _prefill_inputs(83)
    B = inp.spec.block
    k = inp.k.clone()
    nb = inp.spec.n_blocks
    for n in range(1, nb, 2):
        k[:, :, n * B:(n + 1) * B] = k[:, :, (n - 1) * B:n * B]
    inp.k = k
    _say("case: prefill ties, paired key blocks")
    kinds = _prefill_case(inp)
    assert kinds[2] >= 20, kinds


# ---------------------------------------------------------------- decode


def _decode_inputs(seed):
    spec = W.DECODE_128K.with_(batch=2, kv_len=8192, tok_lo=256, tok_hi=2048, stream_local=8)
    return W.make_decode(spec, seed, device=DEV)


def _decode_case(inp):
    spec = inp.spec
    plan = SA.DecodePlan(inp.q, inp.k, inp.v, inp.budget, out_f32=True)
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device=DEV)
    plan.pool(inp.k)
    plan.select(inp.q, inp.k)
    plan.attend(inp.q, inp.k, inp.v, o, lse)
    torch.cuda.synchronize()
    q, k, v = W.to_numpy(inp.q), W.to_numpy(inp.k), W.to_numpy(inp.v)
    gidx, gcnt = plan.block_idx.cpu().numpy(), plan.block_cnt.cpu().numpy()
    oidx, ocnt, sc = O.decode_select(q, k, inp.budget, kmax=plan.kmax, return_scores=True)
    kinds = [0, 0, 0]
    for bi in range(spec.batch):
        for h in range(spec.n_q_heads):
            g = int(inp.budget["granularity"][h])
            nc = -(-spec.kv_len // g)
            c = int(ocnt[bi, h])
            assert int(gcnt[bi, h]) == c
            F = O.forced_blocks(nc, int(inp.budget["n_sink"][h]), int(inp.budget["n_local"][h]))
            kinds[check_row(gidx[bi, h, :c], oidx[bi, h, :c], sc[bi, h], c, F)] += 1
    ro, rl = O.decode_attention(q, k, v, gidx, gcnt, inp.budget["granularity"])
    err, lerr = max_abs(o.cpu().numpy(), ro), max_abs(lse.cpu().numpy(), rl)
    _say("decode rows exempt / gap-pinned / tie-pinned", kinds, "max abs err o", err, "lse", lerr)
    assert err <= TOL_BF16 and lerr <= 1e-4
    return kinds


def test_decode_ties_zero_query():
    """q = 0: every retrieval score is zero; each retrieval head keeps block 0,
    the last block and the lowest-index candidates."""
    inp = _decode_inputs(84)
    inp.q = torch.zeros_like(inp.q)
    _say("case: decode ties, q = 0")
    kinds = _decode_case(inp)
    assert kinds[0] == 0
    assert kinds[2] >= 20, kinds


def test_decode_ties_disjoint_support():
    """q lives on d < D/2 and the keys on d >= D/2: q is orthogonal to every
    pooled key, each product in a score is a signed zero, so every score is
    zero (-0 and +0 are equal)."""
    inp = _decode_inputs(85)
    D = inp.spec.head_dim
    q = inp.q.clone()
    q[..., D // 2:] = 0
    k = inp.k.clone()
    k[..., :D // 2] = 0
    inp.q, inp.k = q, k
    _say("case: decode ties, disjoint support")
    kinds = _decode_case(inp)
    assert kinds[0] == 0
    assert kinds[2] >= 20, kinds


def test_decode_ties_paired_chunks():
    """64-token chunk 2i+1 of the cache a copy of chunk 2i: at every granularity
    (16, 32, 64) the pooled keys, and so the scores, tie in pairs."""
    inp = _decode_inputs(86)
    k = inp.k.clone()
    L = inp.spec.kv_len
    for c in range(1, L // 64, 2):
        k[:, :, c * 64:(c + 1) * 64] = k[:, :, (c - 1) * 64:c * 64]
    inp.k = k
    _say("case: decode ties, paired chunks")
    kinds = _decode_case(inp)
    assert kinds[2] >= 5, kinds
