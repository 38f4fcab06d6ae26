"""Pins for the oracle's attention over gathered blocks (prefill and decode).

The oracle is tied to textbook attention (PyTorch's scaled_dot_product_attention
on the CPU in fp64) when the budget covers every causal block, to closed forms on
hand-built rows, and to invariances any softmax attention must have.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from head_heterogeneous_block_amd import workloads as W


def _full_selection(b, hq, nb):
    idx = np.full((b, hq, nb, nb), -1, dtype=np.int32)
    cnt = np.zeros((b, hq, nb), dtype=np.int32)
    for m in range(nb):
        idx[:, :, m, : m + 1] = np.arange(m + 1)
        cnt[:, :, m] = m + 1
    return idx, cnt


def _sdpa_causal(q, k, v, G):
    qt = torch.from_numpy(O.to_f64(q))
    kt = torch.from_numpy(O.to_f64(k)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(O.to_f64(v)).repeat_interleave(G, dim=1)
    return F.scaled_dot_product_attention(qt, kt, vt, is_causal=True).numpy()


@pytest.mark.parametrize("S,B", [(256, 64), (200, 64)])
def test_full_budget_is_textbook_causal_attention(S, B):
    rng = np.random.default_rng(10)
    b, hq, hkv, D = 2, 4, 2, 32
    q = rng.standard_normal((b, hq, S, D)).astype(np.float32)
    k = rng.standard_normal((b, hkv, S, D)).astype(np.float32)
    v = rng.standard_normal((b, hkv, S, D)).astype(np.float32)
    nb = -(-S // B)
    idx, cnt = _full_selection(b, hq, nb)
    o, lse = O.attention_prefill_gather(q, k, v, idx, cnt, B)
    ref = _sdpa_causal(q, k, v, hq // hkv)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # lse against the library log-sum-exp of the causal logits
    from scipy.special import logsumexp
    for h in range(hq):
        z = (O.to_f64(q[0, h]) @ O.to_f64(k[0, h // 2]).T) / math.sqrt(D)
        z = np.where(np.tril(np.ones((S, S), bool)), z, -np.inf)
        np.testing.assert_allclose(lse[0, h], logsumexp(z, axis=1), rtol=0, atol=1e-12)


def test_full_budget_bf16_inputs_through_selection():
    """Selection with a budget covering every causal block, then attention:
    identical to textbook causal attention on the widened bf16 values."""
    spec = W.LLAMA_32K.with_(seq_len=1024, n_q_heads=8, n_kv_heads=2, head_dim=64, budget_kind="count",
                              counts=(10**6,))
    inp = W.make_prefill(spec, 3)
    q, k, v = (W.to_numpy(t) for t in (inp.q, inp.k, inp.v))
    idx, cnt = O.select_blocks_prefill(q, k, inp.budget, spec.block)
    assert np.all(cnt[0] == np.arange(1, spec.n_blocks + 1)[None, :])
    o, _ = O.attention_prefill_gather(q, k, v, idx, cnt, spec.block)
    np.testing.assert_allclose(o, _sdpa_causal(q, k, v, spec.group), rtol=0, atol=1e-12)


def test_first_row_and_two_key_closed_forms():
    rng = np.random.default_rng(11)
    S, B, D = 128, 64, 16
    q = rng.standard_normal((1, 1, S, D))
    k = rng.standard_normal((1, 1, S, D))
    v = rng.standard_normal((1, 1, S, D))
    idx, cnt = _full_selection(1, 1, 2)
    o, lse = O.attention_prefill_gather(q, k, v, idx, cnt, B)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])  # row 0 sees only key 0
    assert lse[0, 0, 0] == pytest.approx(q[0, 0, 0] @ k[0, 0, 0] / 4.0, abs=1e-14)
    dz = (q[0, 0, 1] @ k[0, 0, 0] - q[0, 0, 1] @ k[0, 0, 1]) / 4.0
    sig = 1.0 / (1.0 + math.exp(-dz))
    np.testing.assert_allclose(o[0, 0, 1], sig * v[0, 0, 0] + (1 - sig) * v[0, 0, 1], atol=1e-14)


def test_one_block_known_logits():
    """Keys built so that a query row sees logits 0, ln 2, ln 3 exactly on the
    three keys it can reach: weights 1/6, 2/6, 3/6."""
    D, B = 4, 4
    S = 8
    q = np.zeros((1, 1, S, D))
    k = np.zeros((1, 1, S, D))
    v = np.zeros((1, 1, S, D))
    q[0, 0, 6] = [2.0, 0, 0, 0]  # scale 1/sqrt(4) = 1/2 -> logit = k[0]
    k[0, 0, 4:7, 0] = [0.0, math.log(2), math.log(3)]
    v[0, 0, 4:7] = np.eye(4)[:3] * 6.0
    idx = np.array([[[[0, -1], [1, -1]]]], dtype=np.int32)  # block 1 selects only itself
    cnt = np.array([[[1, 1]]], dtype=np.int32)
    o, lse = O.attention_prefill_gather(q, k, v, idx, cnt, B)
    np.testing.assert_allclose(o[0, 0, 6], [1.0, 2.0, 3.0, 0.0], atol=1e-14)
    assert lse[0, 0, 6] == pytest.approx(math.log(6.0), abs=1e-14)


def test_invariances_constant_v_shift_permutation_gqa():
    rng = np.random.default_rng(12)
    spec = W.TINY_F32.with_(seq_len=512, n_q_heads=4, n_kv_heads=2, counts=(3, 5))
    inp = W.make_prefill(spec, 12)
    q, k, v = (W.to_numpy(t).astype(np.float64) for t in (inp.q, inp.k, inp.v))
    idx, cnt = O.select_blocks_prefill(q, k, inp.budget, spec.block)
    o, lse = O.attention_prefill_gather(q, k, v, idx, cnt, spec.block)
    # constant V -> output is that constant
    c = rng.standard_normal(spec.head_dim)
    oc, _ = O.attention_prefill_gather(q, k, np.broadcast_to(c, v.shape).copy(), idx, cnt, spec.block)
    np.testing.assert_allclose(oc, np.broadcast_to(c, oc.shape), atol=1e-13)
    # same vector added to every key: equal logit shift per row (large, to test
    # the max subtraction) -> output unchanged
    w = rng.standard_normal(spec.head_dim)
    w *= 640.0 / np.linalg.norm(w)  # logit shifts of order +-100
    shift = (q[0] @ w) / math.sqrt(spec.head_dim)
    assert np.abs(shift).max() > 80.0
    os_, _ = O.attention_prefill_gather(q, k + w, v, idx, cnt, spec.block)
    np.testing.assert_allclose(os_, o, atol=1e-9)
    # any order of the selected blocks in the index table
    perm = idx.copy()
    for h in range(spec.n_q_heads):
        for m in range(spec.n_blocks):
            c_ = cnt[0, h, m]
            perm[0, h, m, :c_] = perm[0, h, m, :c_][::-1]
    op, _ = O.attention_prefill_gather(q, k, v, perm, cnt, spec.block)
    np.testing.assert_allclose(op, o, atol=1e-13)
    # GQA == multi-head attention with each KV head repeated for its group
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    om, _ = O.attention_prefill_gather(q, kr, vr, idx, cnt, spec.block)
    np.testing.assert_allclose(om, o, atol=1e-15)


@pytest.mark.parametrize("base,S", [(W.TINY_F32, None), (W.LLAMA_32K, 2048)], ids=["tiny-f32", "llama-2k"])
def test_gather_form_equals_dense_masked_form(base, S):
    spec = base
    if S:
        spec = spec.with_(seq_len=S, n_q_heads=8, n_kv_heads=2)
    inp = W.make_prefill(spec, 20 + W.seed_of(base) - 1000)
    q, k, v = (W.to_numpy(t) for t in (inp.q, inp.k, inp.v))
    idx, cnt = O.select_blocks_prefill(q, k, inp.budget, spec.block)
    o1, l1 = O.attention_prefill_gather(q, k, v, idx, cnt, spec.block)
    o2, l2 = O.attention_prefill_dense_masked(q, k, v, idx, cnt, spec.block)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_decode_full_budget_is_library_attention():
    spec = W.DECODE_128K.with_(batch=2, kv_len=1024, n_streaming=0, tok_lo=1024, tok_hi=1025, n_hot=2)
    inp = W.make_decode(spec, 9)
    q, k, v = (W.to_numpy(t) for t in (inp.q, inp.k, inp.v))
    idx, cnt = O.decode_select(q, k, inp.budget)
    nc = spec.kv_len // inp.budget["granularity"]
    assert np.all(cnt == nc[None, :])
    o, lse = O.decode_attention(q, k, v, idx, cnt, inp.budget["granularity"])
    qt = torch.from_numpy(O.to_f64(q))[:, :, None, :]
    kt = torch.from_numpy(O.to_f64(k)).repeat_interleave(spec.group, dim=1)
    vt = torch.from_numpy(O.to_f64(v)).repeat_interleave(spec.group, dim=1)
    ref = F.scaled_dot_product_attention(qt, kt, vt)[:, :, 0, :].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    from scipy.special import logsumexp
    z = torch.einsum("bhd,bhld->bhl", qt[:, :, 0, :], kt).numpy() / math.sqrt(spec.head_dim)
    np.testing.assert_allclose(lse, logsumexp(z, axis=-1), rtol=0, atol=1e-12)


def test_decode_gather_equals_dense_mask():
    spec = W.DECODE_128K.with_(batch=2, kv_len=4096, n_streaming=3, tok_lo=256, tok_hi=1024, stream_local=8)
    inp = W.make_decode(spec, 13)
    q, k, v = (W.to_numpy(t) for t in (inp.q, inp.k, inp.v))
    idx, cnt = O.decode_select(q, k, inp.budget)
    o, lse = O.decode_attention(q, k, v, idx, cnt, inp.budget["granularity"])
    mask = np.zeros((spec.batch, spec.n_q_heads, spec.kv_len), bool)
    for bi in range(spec.batch):
        for h in range(spec.n_q_heads):
            g = inp.budget["granularity"][h]
            for n in idx[bi, h, : cnt[bi, h]]:
                mask[bi, h, n * g:(n + 1) * g] = True
    o2, l2 = O.decode_attention_dense(q, k, v, mask)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(lse, l2, atol=1e-12)
