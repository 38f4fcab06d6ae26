"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Bars: block indices bit-exact on every pinned row (score gap > 1e-4 relative,
ties to the lowest index), valid on near-tie rows; LPT schedules bit-exact;
attention max-abs error <= 1e-5 for fp32 inputs and <= 1e-2 for bf16 inputs
(fp32 output), bf16 output within 1e-2 + half a bf16 ulp of the oracle value.
"""

import numpy as np
import pytest
import torch

import oracle as O
from head_heterogeneous_block_amd import workloads as W

from gpu_helpers import (bf16_half_ulp, check_prefill_selection, check_row, max_abs, prefill_gpu, to_host)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from head_heterogeneous_block_amd import sparse_attn as SA  # noqa: E402  (fails loudly if not built)

DEV = "cuda:0"
TOL_F32 = 1e-5
TOL_BF16 = 1e-2


def _say(*a):
    print(*a, flush=True)


def _bud_sub(budget, heads):
    return {k: np.asarray(v)[heads] for k, v in budget.items()}


# ---------------------------------------------------------------- prefill, all rows


@pytest.mark.parametrize("schedule", ["natural", "lpt", "queue"])
def test_prefill_config0_fp32_all_rows(schedule):
    spec = W.TINY_F32
    inp = W.make_prefill(spec, W.seed_of(W.TINY_F32), device=DEV)
    _say("case: config0 fp32", schedule)
    # queue: 3 workgroups over the queue in 8 XCD partitions (one KV group,
    # so seven partitions are empty and every workgroup walks them)
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins={"natural": 0, "lpt": 8, "queue": 3}[schedule],
                                         queue=schedule == "queue")
    q, k, v = to_host(inp)
    oidx, ocnt, scores = O.select_blocks_prefill(q, k, inp.budget, spec.block, kmax=plan.kmax, return_scores=True)
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    pinned, exempt = check_prefill_selection(gidx, gcnt, oidx, ocnt, scores, inp.budget)
    _say("pinned", pinned, "exempt", exempt)
    assert pinned >= 0.9 * (pinned + exempt)
    ro, rl = O.attention_prefill_gather(q, k, v, gidx, gcnt, spec.block)
    err = max_abs(o.cpu().numpy(), ro)
    lerr = max_abs(lse.cpu().numpy(), rl)
    _say("max abs err o", err, "lse", lerr)
    assert err <= TOL_F32 and lerr <= TOL_F32
    if schedule == "lpt":
        # the oracle's LPT bins, each walked in item order (the plan's default)
        ref = O.lpt_schedule(plan.counts.reshape(-1).tolist(), 8)
        off = ref[1]
        want = np.concatenate([np.sort(ref[2][off[b]:off[b + 1]]) for b in range(8)])
        np.testing.assert_array_equal(plan.bin_offsets.cpu().numpy(), off)
        np.testing.assert_array_equal(plan.items_by_bin.cpu().numpy(), want)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("schedule", ["natural", "queue"])
def test_prefill_fp32_batched_ragged(schedule, D):
    """The fp32 path (both head sizes) over two sequences of a ragged length
    (not a multiple of the 64-token block): batch strides, the partial last
    block, and the schedule's (sequence, KV head) groups."""
    spec = W.TINY_F32.with_(batch=2, seq_len=1000, head_dim=D)
    inp = W.make_prefill(spec, 91, device=DEV)
    _say("case: fp32 batched ragged", schedule, "D", D)
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins={"natural": 0, "queue": 5}[schedule],
                                         queue=schedule == "queue", queue_group="kv_tiers")
    q, k, v = to_host(inp)
    oidx, ocnt, scores = O.select_blocks_prefill(q, k, inp.budget, spec.block, kmax=plan.kmax, return_scores=True)
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    pinned, exempt = check_prefill_selection(gidx, gcnt, oidx, ocnt, scores, inp.budget)
    _say("pinned", pinned, "exempt", exempt)
    assert pinned >= 0.9 * (pinned + exempt)
    ro, rl = O.attention_prefill_gather(q, k, v, gidx, gcnt, spec.block)
    err = max_abs(o.cpu().numpy(), ro)
    lerr = max_abs(lse.cpu().numpy(), rl)
    _say("max abs err o", err, "lse", lerr)
    assert err <= TOL_F32 and lerr <= TOL_F32


PREFILL_SHAPES = [
    # name, overrides
    ("llama-2k", dict(seq_len=2048, n_q_heads=8, n_kv_heads=2)),
    ("llama-ragged", dict(seq_len=2000, n_q_heads=8, n_kv_heads=2)),
    ("d64-b128", dict(seq_len=1536, n_q_heads=4, n_kv_heads=1, head_dim=64)),
    ("b64", dict(seq_len=1500, n_q_heads=4, n_kv_heads=2, block=64)),
    ("d64-b64", dict(seq_len=1300, n_q_heads=4, n_kv_heads=1, head_dim=64, block=64)),
    ("mha-3heads", dict(seq_len=1100, n_q_heads=3, n_kv_heads=3)),  # one query head per KV head
    ("one-block", dict(seq_len=100, n_q_heads=2, n_kv_heads=1)),
    ("tiny-17", dict(seq_len=17, n_q_heads=2, n_kv_heads=1)),
    ("one-token", dict(seq_len=1, n_q_heads=4, n_kv_heads=2)),
    # several sequences: the batch strides of Q, K, V and O, the key-norm
    # table's rows and the schedule's (sequence, KV head) groups
    ("batch3-ragged", dict(batch=3, seq_len=1000, n_q_heads=4, n_kv_heads=1)),
    ("batch2-b64", dict(batch=2, seq_len=700, n_q_heads=4, n_kv_heads=2, block=64)),
]


@pytest.mark.parametrize("name,over", PREFILL_SHAPES, ids=[s[0] for s in PREFILL_SHAPES])
@pytest.mark.parametrize("sched", ["natural", "bins37", "queue23", "queue23x1"])
def test_prefill_bf16_all_rows(name, over, sched):
    spec = W.LLAMA_32K.with_(**over)
    inp = W.make_prefill(spec, 77, device=DEV)
    _say("case:", name, "schedule", sched)
    n_bins = {"natural": 0, "bins37": 37, "queue23": 23, "queue23x1": 23}[sched]
    # queue23: the tiered queue cut into 8 partitions (the default beyond 256
    # query blocks); queue23x1: one tiered queue
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins=n_bins, queue=sched.startswith("queue"),
                                         queues=1 if sched.endswith("x1") else 8, queue_group="kv_tiers")
    q, k, v = to_host(inp)
    oidx, ocnt, scores = O.select_blocks_prefill(q, k, inp.budget, spec.block, kmax=plan.kmax, return_scores=True)
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    pinned, exempt = check_prefill_selection(gidx, gcnt, oidx, ocnt, scores, inp.budget)
    _say("pinned", pinned, "exempt", exempt)
    ro, rl = O.attention_prefill_gather(q, k, v, gidx, gcnt, spec.block)
    err = max_abs(o.cpu().numpy(), ro)
    lerr = max_abs(lse.cpu().numpy(), rl)
    _say("max abs err o", err, "lse", lerr)
    assert err <= TOL_BF16 and lerr <= TOL_BF16


def test_prefill_bf16_output_and_determinism():
    spec = W.LLAMA_32K.with_(seq_len=2048 + 128, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, 5, device=DEV)
    idx, cnt, o16, _, plan = prefill_gpu(inp, out_f32=False, with_lse=False)
    q, k, v = to_host(inp)
    ro, _ = O.attention_prefill_gather(q, k, v, idx.cpu().numpy(), cnt.cpu().numpy(), spec.block)
    got = o16.float().cpu().numpy()
    bound = TOL_BF16 + bf16_half_ulp(ro)
    assert np.all(np.abs(got - ro) <= bound)
    _, _, o16b, _, _ = prefill_gpu(inp, out_f32=False, with_lse=False)
    assert torch.equal(o16, o16b), "two runs differ"


def test_prefill_schedules_bitwise_equal():
    """Every tile is computed by one workgroup with the same arithmetic whatever
    the schedule: outputs must be identical bit for bit."""
    spec = W.LLAMA_32K.with_(seq_len=4096, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, 9, device=DEV)
    outs = []
    for n_bins in (0, 1, 64, 512, 97):
        _say("schedule", n_bins)
        _, _, o, lse, _ = prefill_gpu(inp, n_bins=n_bins)
        outs.append((o, lse))
    # two-level (cache-partition) placement, assignment-order bins, and the
    # work queue with one worker, some, and more workers than tiles (each
    # queue plan attends twice: the counters are reset by every call); the
    # queue cut into partitions (2 KV groups here, so most partitions are
    # empty), one worker walking all 16 of them, more workers than tiles
    for kw in (dict(xcd_groups=8, xcd_chunk=4), dict(bin_order="lpt"), dict(queue=True),
               dict(queue=True, n_bins=1), dict(queue=True, n_bins=5000), dict(queue=True, queue_group="kv"),
               dict(queue=True, queue_group="flat"), dict(queue=True, queue_group="head"),
               dict(queue=True, queue_group="kv_tiers"), dict(queue=True, queue_group="kv_tiers", queues=1),
               dict(queue=True, queue_group="kv_tiers", queues=1, n_bins=1),
               dict(queue=True, queue_group="kv_tiers", queue_chunk=3),
               dict(queue=True, queue_group="kv_tiers", queues=3, n_bins=5),
               dict(queue=True, queue_group="kv_tiers", queues=16, n_bins=1),
               dict(queue=True, queue_group="kv_tiers", queues=16, n_bins=5000),
               dict(queue=True, queue_group="kv_tiers", queues=2, n_bins=2)):
        _say("schedule", kw)
        kw = dict(kw)
        nb = kw.pop("n_bins", 64)
        plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=nb, out_f32=True, **kw)
        plan.select(inp.q, inp.k)
        for _ in range(2 if plan.queue else 1):
            o = torch.full(inp.q.shape, float("nan"), dtype=torch.float32, device=DEV)
            lse = torch.full(inp.q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
            plan.attend(inp.q, inp.k, inp.v, o, lse)
            torch.cuda.synchronize()
            outs.append((o, lse))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


# ---------------------------------------------------------------- prefill, full sizes


@pytest.mark.parametrize("spec", [W.LLAMA_32K, W.LLAMA_128K, W.QWEN_64K], ids=lambda s: s.name)
def test_prefill_full_size_sampled(spec):
    _say("case: full-size workload", spec.name)
    inp = W.make_prefill(spec, W.seed_of(spec), device=DEV)
    n_bins = 512
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins=n_bins, queue=True)  # the benchmark's launch
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    np.testing.assert_array_equal(gcnt, plan.counts)
    G = spec.group
    nb = spec.n_blocks
    heads = [0, spec.n_q_heads // 2 + 1, spec.n_q_heads - 1]
    q, k, v = W.to_numpy(inp.q[:, heads]), None, None
    kv_heads = [h // G for h in heads]
    k = W.to_numpy(inp.k[:, kv_heads])
    vv = W.to_numpy(inp.v[:, kv_heads])
    # selection of the sampled heads, every row (each head paired with its own KV head)
    for i, h in enumerate(heads):
        sub = _bud_sub(inp.budget, [h])
        oidx, ocnt, sc = O.select_blocks_prefill(q[:, [i]], k[:, [i]], sub, spec.block, kmax=plan.kmax,
                                                 return_scores=True)
        pinned, exempt = check_prefill_selection(gidx[:, [h]], gcnt[:, [h]], oidx, ocnt, sc, sub)
        _say("head", h, "pinned", pinned, "exempt", exempt)
        assert pinned >= 0.9 * (pinned + exempt)
    # attention on sampled tiles, oracle over the GPU's block lists
    rng = np.random.default_rng(W.seed_of(spec))
    ms = sorted(set([0, 1, nb - 1] + rng.integers(0, nb, 5).tolist()))
    tiles = [(0, i, m) for i in range(len(heads)) for m in ms]
    sub_idx = gidx[:, heads]
    sub_cnt = gcnt[:, heads]
    ro, rl = O.attention_prefill_gather(q, k, vv, sub_idx, sub_cnt, spec.block, tiles=tiles)
    og = o[:, heads].cpu().numpy()
    lg = lse[:, heads].cpu().numpy()
    worst = 0.0
    for (bi, i, m) in tiles:
        rows = slice(m * spec.block, min(spec.seq_len, (m + 1) * spec.block))
        worst = max(worst, max_abs(og[bi, i, rows], ro[bi, i, rows]), max_abs(lg[bi, i, rows], rl[bi, i, rows]))
    _say("max abs err over", len(tiles), "tiles:", worst)
    assert worst <= TOL_BF16
    assert torch.isfinite(o).all()


def test_prefill_long_rows_sampled():
    """Rows longer than 1024 blocks (131072 + 37 tokens in 64-token blocks: 2049
    candidates in the last row, ragged): the selection keeps fewer rows per
    workgroup there, and the attention reads block ids and key-norm rows beyond
    1024.  Every row's selection against the oracle; attention on tiles on
    both sides of 1024 and at the ragged end, on the benchmark's launch (the
    work queue in XCD partitions)."""
    spec = W.LLAMA_32K.with_(seq_len=2048 * 64 + 37, block=64, n_q_heads=2, n_kv_heads=1)
    _say("case: long rows", spec)
    inp = W.make_prefill(spec, 61, device=DEV)
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins=512, queue=True)
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    q, k, v = to_host(inp)
    oidx, ocnt, sc = O.select_blocks_prefill(q, k, inp.budget, spec.block, kmax=plan.kmax, return_scores=True)
    pinned, exempt = check_prefill_selection(gidx, gcnt, oidx, ocnt, sc, inp.budget)
    _say("pinned", pinned, "exempt", exempt)
    assert pinned >= 0.9 * (pinned + exempt)
    tiles = [(0, h, m) for h in range(2) for m in (0, 1, 1023, 1024, 1025, 2047, 2048)]
    ro, rl = O.attention_prefill_gather(q, k, v, gidx, gcnt, spec.block, tiles=tiles)
    og, lg = o.cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    for (bi, h, m) in tiles:
        rows = slice(m * spec.block, min(spec.seq_len, (m + 1) * spec.block))
        worst = max(worst, max_abs(og[bi, h, rows], ro[bi, h, rows]), max_abs(lg[bi, h, rows], rl[bi, h, rows]))
    _say("max abs err over", len(tiles), "tiles:", worst)
    assert worst <= TOL_BF16
    assert torch.isfinite(o).all()


# ---------------------------------------------------------------- decode


def _decode_gpu(inp, out_f32=True):
    q, k, v = inp.q, inp.k, inp.v
    plan = SA.DecodePlan(q, k, v, inp.budget, out_f32=out_f32)
    o = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    plan.pool(k)
    plan.select(q, k)
    plan.attend(q, k, v, o, lse)
    torch.cuda.synchronize()
    return plan, o, lse


def _check_decode(inp, plan, o, lse, seqs):
    spec = inp.spec
    gidx, gcnt = plan.block_idx.cpu().numpy(), plan.block_cnt.cpu().numpy()
    np.testing.assert_array_equal(gcnt, np.broadcast_to(plan.counts, gcnt.shape))
    q = W.to_numpy(inp.q[seqs])
    k = W.to_numpy(inp.k[seqs])
    v = W.to_numpy(inp.v[seqs])
    oidx, ocnt, sc = O.decode_select(q, k, inp.budget, kmax=plan.kmax, return_scores=True)
    pinned = exempt = 0
    for i, bi in enumerate(seqs):
        for h in range(spec.n_q_heads):
            g = int(inp.budget["granularity"][h])
            nc = -(-spec.kv_len // g)
            c = int(ocnt[i, h])
            assert int(gcnt[bi, h]) == c
            F = O.forced_blocks(nc, int(inp.budget["n_sink"][h]), int(inp.budget["n_local"][h]))
            if check_row(gidx[bi, h, :c], oidx[i, h, :c], sc[i, h], c, F):
                pinned += 1
            else:
                exempt += 1
    _say("decode pinned", pinned, "exempt", exempt)
    ro, rl = O.decode_attention(q, k, v, gidx[seqs], gcnt[seqs], inp.budget["granularity"])
    err = max_abs(o[seqs].cpu().numpy(), ro)
    lerr = max_abs(lse[seqs].cpu().numpy(), rl)
    _say("decode max abs err o", err, "lse", lerr)
    assert err <= TOL_BF16 and lerr <= TOL_BF16


@pytest.mark.parametrize("L", [8192, 8192 + 40, 1000])
def test_decode_reduced_all(L):
    spec = W.DECODE_128K.with_(batch=3, kv_len=L, tok_lo=256, tok_hi=2048, stream_local=16)
    _say("case: decode L", L)
    inp = W.make_decode(spec, 31, device=DEV)
    plan, o, lse = _decode_gpu(inp)
    _check_decode(inp, plan, o, lse, list(range(spec.batch)))


def test_custom_softmax_scale():
    """A softmax scale other than 1/sqrt(D) (0.05; 1/sqrt(128) = 0.088), prefill
    and decode: selections and outputs against the oracle run with the same
    scale.  (The top-k order does not depend on a positive scale; the
    attention's exponent does.)"""
    scale = 0.05
    spec = W.LLAMA_32K.with_(seq_len=1500, n_q_heads=4, n_kv_heads=2)
    _say("case: scale", scale, "prefill")
    inp = W.make_prefill(spec, 83, device=DEV)
    plan = SA.PrefillPlan(inp.q, inp.k, inp.v, inp.budget, spec.block, n_bins=16, out_f32=True, queue=True,
                          queue_group="kv_tiers", scale=scale)
    o = torch.empty(inp.q.shape, dtype=torch.float32, device=DEV)
    lse = torch.empty(inp.q.shape[:3], dtype=torch.float32, device=DEV)
    plan.select(inp.q, inp.k)
    plan.attend(inp.q, inp.k, inp.v, o, lse)
    torch.cuda.synchronize()
    q, k, v = to_host(inp)
    gidx, gcnt = plan.block_idx.cpu().numpy(), plan.block_cnt.cpu().numpy()
    oidx, ocnt, sc = O.select_blocks_prefill(q, k, inp.budget, spec.block, kmax=plan.kmax, scale=scale,
                                             return_scores=True)
    pinned, exempt = check_prefill_selection(gidx, gcnt, oidx, ocnt, sc, inp.budget)
    assert pinned >= 0.9 * (pinned + exempt)
    ro, rl = O.attention_prefill_gather(q, k, v, gidx, gcnt, spec.block, scale=scale)
    err, lerr = max_abs(o.cpu().numpy(), ro), max_abs(lse.cpu().numpy(), rl)
    _say("prefill max abs err o", err, "lse", lerr)
    assert err <= TOL_BF16 and lerr <= TOL_BF16
    # decode
    dspec = W.DECODE_128K.with_(batch=2, kv_len=4096 + 24, tok_lo=256, tok_hi=1024, stream_local=8)
    _say("case: scale", scale, "decode")
    dinp = W.make_decode(dspec, 84, device=DEV)
    dplan = SA.DecodePlan(dinp.q, dinp.k, dinp.v, dinp.budget, out_f32=True, scale=scale)
    do = torch.empty(dinp.q.shape, dtype=torch.float32, device=DEV)
    dl = torch.empty(dinp.q.shape[:2], dtype=torch.float32, device=DEV)
    dplan.pool(dinp.k)
    dplan.select(dinp.q, dinp.k)
    dplan.attend(dinp.q, dinp.k, dinp.v, do, dl)
    torch.cuda.synchronize()
    dq, dk, dv = W.to_numpy(dinp.q), W.to_numpy(dinp.k), W.to_numpy(dinp.v)
    dgidx, dgcnt = dplan.block_idx.cpu().numpy(), dplan.block_cnt.cpu().numpy()
    ro, rl = O.decode_attention(dq, dk, dv, dgidx, dgcnt, dinp.budget["granularity"], scale=scale)
    err, lerr = max_abs(do.cpu().numpy(), ro), max_abs(dl.cpu().numpy(), rl)
    _say("decode max abs err o", err, "lse", lerr)
    assert err <= TOL_BF16 and lerr <= TOL_BF16


def test_decode_long_cache():
    """A cache longer than the 131072-token workload (200003 tokens): the heads
    at granularity 16 score 12501 pooled keys instead of at most 8192, so the
    top-k runs its widest shape (1024 threads, 16 keys each); every row against
    the oracle, outputs within the bound."""
    spec = W.DECODE_128K.with_(batch=1, kv_len=200003)
    _say("case: decode long cache", spec.kv_len)
    inp = W.make_decode(spec, 47, device=DEV)
    assert 16 in {int(g) for g in inp.budget["granularity"]}
    plan, o, lse = _decode_gpu(inp)
    _check_decode(inp, plan, o, lse, [0])


@pytest.mark.parametrize("name,over", [
    ("d64", dict(head_dim=64)),
    ("gqa8", dict(n_q_heads=16, n_kv_heads=2, n_streaming=4)),
    ("mha", dict(n_q_heads=6, n_kv_heads=6, n_streaming=2)),
    ("tiny-L", dict(kv_len=40, tok_lo=16, tok_hi=64, stream_local=4)),
], ids=["d64", "gqa8", "mha", "tiny-L"])
def test_decode_bf16_shapes(name, over):
    """The bf16 MFMA decode path at other head sizes and group sizes, and a
    cache shorter than one 64-token block (every head keeps all its blocks)."""
    base = dict(batch=2, kv_len=4096 + 24, tok_lo=256, tok_hi=1024, stream_local=8)
    base.update(over)
    spec = W.DECODE_128K.with_(**base)
    _say("case: decode bf16", name)
    inp = W.make_decode(spec, 33, device=DEV)
    plan, o, lse = _decode_gpu(inp)
    _check_decode(inp, plan, o, lse, list(range(spec.batch)))


def test_decode_bf16_output():
    """bf16 output: within the fp32 tolerance plus half a bf16 ulp of the value."""
    spec = W.DECODE_128K.with_(batch=2, kv_len=8192, tok_lo=256, tok_hi=2048, stream_local=16)
    inp = W.make_decode(spec, 34, device=DEV)
    plan, o, lse = _decode_gpu(inp, out_f32=False)
    assert o.dtype == torch.bfloat16
    q, k, v = W.to_numpy(inp.q), W.to_numpy(inp.k), W.to_numpy(inp.v)
    gidx, gcnt = plan.block_idx.cpu().numpy(), plan.block_cnt.cpu().numpy()
    ro, _ = O.decode_attention(q, k, v, gidx, gcnt, inp.budget["granularity"])
    og = o.float().cpu().numpy()
    assert np.all(np.abs(og - ro) <= TOL_BF16 + bf16_half_ulp(ro))


def test_decode_pooled_key_cache():
    """The pooled-key cache (the Index step) against the oracle's block means:
    one fp32 array [b][Hkv][ceil(L/g)][D] per granularity the scoring heads use,
    ascending, packed back to back."""
    spec = W.DECODE_128K.with_(batch=2, kv_len=4096 + 24, tok_lo=256, tok_hi=1024, stream_local=8)
    inp = W.make_decode(spec, 35, device=DEV)
    plan = SA.DecodePlan(inp.q, inp.k, inp.v, inp.budget)
    plan.pool(inp.k)
    torch.cuda.synchronize()
    got_all = plan.k_pooled.cpu().numpy()
    k = W.to_numpy(inp.k)
    grans = sorted({int(inp.budget["granularity"][h]) for h in range(spec.n_q_heads) if not inp.budget["streaming"][h]})
    off = 0
    for g in grans:
        nc = -(-spec.kv_len // g)
        n = spec.batch * spec.n_kv_heads * nc * spec.head_dim
        got = got_all[off:off + n].reshape(spec.batch, spec.n_kv_heads, nc, spec.head_dim)
        ref = O.pool_blocks(k, g)
        err = float(np.max(np.abs(got - ref)))
        _say("pooled g", g, "max abs err", err)
        assert err <= 1e-5  # fp32 sums of <= 64 bf16 values
        off += n


def test_decode_gqa8_fp32():
    spec = W.DECODE_128K.with_(dtype="f32", batch=2, n_q_heads=16, n_kv_heads=2, kv_len=4096, tok_lo=256,
                              tok_hi=1024, stream_local=8, n_streaming=4)
    inp = W.make_decode(spec, 32, device=DEV)
    plan, o, lse = _decode_gpu(inp)
    _check_decode(inp, plan, o, lse, [0, 1])


def test_decode_full_size_sampled():
    spec = W.DECODE_128K
    _say("case: full decode config")
    inp = W.make_decode(spec, W.seed_of(W.DECODE_128K), device=DEV)
    plan, o, lse = _decode_gpu(inp)
    _check_decode(inp, plan, o, lse, [0, 9])
    assert torch.isfinite(o).all()
    # determinism: a second step is bitwise identical
    o2 = torch.empty_like(o)
    plan.select(inp.q, inp.k)
    plan.attend(inp.q, inp.k, inp.v, o2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


# ---------------------------------------------------------------- degenerate budgets


def test_prefill_full_budget_is_dense_causal_attention():
    """A ratio of 1 keeps every causal block: the selection is 0..m for every
    row and the output is dense causal attention (torch's fp64 SDPA on the CPU,
    K/V repeated over the GQA group), ragged tail included."""
    spec = W.LLAMA_32K.with_(seq_len=2048 + 100, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, 61, device=DEV)
    inp.budget["ratio_q16"][:] = 65536
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins=64, queue=True)
    nb = spec.n_blocks
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for m in range(nb):
        assert np.all(gcnt[:, :, m] == m + 1)
        assert np.all(gidx[:, :, m, :m + 1] == np.arange(m + 1))
    q, k, v = (torch.from_numpy(O.to_f64(x)) for x in to_host(inp))
    G = spec.n_q_heads // spec.n_kv_heads
    ref = torch.nn.functional.scaled_dot_product_attention(q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1),
                                                           is_causal=True).numpy()
    err = max_abs(o.cpu().numpy(), ref)
    _say("full budget: max abs err vs dense causal attention", err)
    assert err <= TOL_BF16


def test_prefill_minimal_budget_keeps_sink_and_diagonal():
    """A budget of two blocks keeps exactly the sink and the diagonal block."""
    spec = W.LLAMA_32K.with_(seq_len=1536, n_q_heads=4, n_kv_heads=1)
    inp = W.make_prefill(spec, 62, device=DEV)
    inp.budget["ratio_q16"][:] = 0
    inp.budget["min_blocks"][:] = 2
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins=16, queue=True)
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    assert np.all(gcnt[:, :, 0] == 1) and np.all(gidx[:, :, 0, 0] == 0)
    for m in range(1, spec.n_blocks):
        assert np.all(gcnt[:, :, m] == 2)
        assert np.all(gidx[:, :, m, 0] == 0) and np.all(gidx[:, :, m, 1] == m)
    q, k, v = to_host(inp)
    ro, rl = O.attention_prefill_gather(q, k, v, gidx, gcnt, spec.block)
    err = max_abs(o.cpu().numpy(), ro)
    _say("minimal budget: max abs err", err)
    assert err <= TOL_BF16


# ---------------------------------------------------------------- wide logits


@pytest.mark.parametrize("qmul", [3.0, 4.0, 6.0])
def test_prefill_with_wide_logits(qmul):
    """Q scaled by 3-6 makes each row's softmax sharp: one key often holds most
    of a row's weight and the lazily raised running maximum moves inside tiles
    (rescaling O and l).  Output within 1e-2 and lse within 1e-4 of the oracle,
    like every other bf16 case.  The probabilities are rounded to bf16 for the
    P V MFMAs, and the normaliser sums those same rounded values, so the output
    stays a convex combination of V rows; lse comes from the unrounded sum."""
    spec = W.LLAMA_32K.with_(seq_len=2048 + 64, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, 71, device=DEV)
    inp.q = (inp.q.float() * qmul).to(inp.q.dtype)
    _say("case: prefill wide logits, Q x", qmul)
    idx, cnt, o, lse, plan = prefill_gpu(inp, n_bins=32, queue=True)
    q, k, v = to_host(inp)
    gidx, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    ro, rl = O.attention_prefill_gather(q, k, v, gidx, gcnt, spec.block)
    err, lerr = max_abs(o.cpu().numpy(), ro), max_abs(lse.cpu().numpy(), rl)
    _say("prefill wide logits: max abs err o", err, "lse", lerr, "lse range", float(rl.min()), float(rl.max()))
    assert lerr <= 1e-4
    assert err <= TOL_BF16
    # the same tiles without lse (the kernel variant that keeps one sum)
    o2 = torch.empty_like(o)
    plan.attend(inp.q, inp.k, inp.v, o2, None)
    torch.cuda.synchronize()
    assert torch.equal(o2, o)


@pytest.mark.parametrize("qmul", [3.0, 4.0, 6.0])
def test_decode_with_wide_logits(qmul):
    """Decode with Q scaled by 3-6 (sharp softmax): output within 1e-2, lse
    within 1e-4 of the oracle.  The chunk partials carry both the rounded-P sum
    (normaliser of o) and the unrounded one (lse)."""
    dspec = W.DECODE_128K.with_(batch=2, kv_len=4096 + 24, tok_lo=256, tok_hi=1024, stream_local=8)
    din = W.make_decode(dspec, 72, device=DEV)
    din.q = (din.q.float() * qmul).to(din.q.dtype)
    _say("case: decode wide logits, Q x", qmul)
    dplan, do, dl = _decode_gpu(din)
    gidx, gcnt = dplan.block_idx.cpu().numpy(), dplan.block_cnt.cpu().numpy()
    qd, kd, vd = W.to_numpy(din.q), W.to_numpy(din.k), W.to_numpy(din.v)
    ro, rl = O.decode_attention(qd, kd, vd, gidx, gcnt, din.budget["granularity"])
    err, lerr = max_abs(do.cpu().numpy(), ro), max_abs(dl.cpu().numpy(), rl)
    _say("decode wide logits: max abs err o", err, "lse", lerr)
    assert lerr <= 1e-4
    assert err <= TOL_BF16
