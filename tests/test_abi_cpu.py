"""Host-side tests of the C-ABI library (no GPU needed).

The library loads, exports every function include/sparse_attn.h declares, and
its host-only entry points agree with the oracle: the greedy longest-load-first
schedule bit for bit, the per-row block counts of the budget rule exactly.
Argument validation returns error codes before anything touches a device.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from head_heterogeneous_block_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SA = pytest.importorskip("head_heterogeneous_block_amd.sparse_attn", reason="library not built", exc_type=ImportError)


def _header_functions():
    text = open(os.path.join(ROOT, "include", "sparse_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = _header_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(SA.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(SA.EXPORTED) == names


def test_version_and_error_text():
    assert SA.sa_version() >= 10000
    with pytest.raises(SA.SaError) as e:
        SA.sa_lpt_schedule([1, 2], 0)
    assert e.value.status == SA.SA_ERR_INVALID_ARG and "n_bins" in str(e.value)


@pytest.mark.parametrize("seed", range(6))
def test_lpt_matches_oracle_bit_exact(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 3000))
    bins = int(rng.integers(1, 700))
    loads = rng.integers(0, 50, size=n) if seed % 2 else np.exp(rng.uniform(0, 6, n)).astype(np.int64)
    got = SA.sa_lpt_schedule(loads, bins)
    ref = O.lpt_schedule(loads.tolist(), bins)
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)


def test_lpt_golden_and_negative_load():
    _, off, items, load = SA.sa_lpt_schedule([31, 58, 81, 100], 2)
    assert items.tolist() == [3, 0, 2, 1] and off.tolist() == [0, 2, 4] and load.tolist() == [131, 139]
    with pytest.raises(SA.SaError):
        SA.sa_lpt_schedule([3, -1], 2)


def test_lpt_order_bins_keeps_bins_and_sorts():
    """Reordering inside the bins: same item set per bin (so the same bin
    loads), ascending inside each bin; bad offsets are rejected."""
    rng = np.random.default_rng(5)
    loads = rng.integers(1, 40, size=777)
    bin_of, off, items, load = SA.sa_lpt_schedule(loads, 37)
    got = SA.sa_lpt_order_bins(off, items)
    for b in range(37):
        seg, ref = got[off[b]:off[b + 1]], items[off[b]:off[b + 1]]
        assert seg.tolist() == sorted(ref.tolist())
        assert int(loads[seg].sum()) == int(load[b])
        assert np.all(bin_of[seg] == b)
    with pytest.raises(SA.SaError):
        SA.sa_lpt_order_bins(np.array([0, 5, 3], np.int32), items)


@pytest.mark.parametrize("seed", range(4))
def test_lpt_queue_order(seed):
    """Work-queue order: a permutation, groups ascending, inside a group the
    loads do not increase and equal loads keep item order (the same order a
    stable lexicographic sort on (group, -load) gives)."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(0, 5000))
    loads = rng.integers(0, 40, size=n)
    groups = np.sort(rng.integers(0, 9, size=n)) if seed % 2 else rng.integers(0, 9, size=n)
    order = SA.sa_lpt_queue_order(loads, groups)
    assert sorted(order.tolist()) == list(range(n))
    g, l = groups[order], loads[order]
    assert np.all(np.diff(g) >= 0)
    same = np.diff(g) == 0
    assert np.all(np.diff(l)[same] <= 0)
    ties = same & (np.diff(l) == 0)
    assert np.all(np.diff(order)[ties] > 0)
    np.testing.assert_array_equal(order, np.lexsort((-loads, groups)))
    # no groups: plain longest first
    np.testing.assert_array_equal(SA.sa_lpt_queue_order(loads), np.argsort(-loads, kind="stable"))
    with pytest.raises(SA.SaError):
        SA.sa_lpt_queue_order([1, -2, 3])


@pytest.mark.parametrize("seed", range(4))
def test_lpt_grouped_is_two_oracle_placements(seed):
    """Two-level placement = the oracle's LPT of chunk loads onto groups, then
    the oracle's LPT of each group's items (in item order) onto its bins, bin
    b of group g being b * n_groups + g."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 900))
    n_chunks = int(rng.integers(1, 40))
    n_groups = int(rng.integers(1, 9))
    per = int(rng.integers(1, 9))
    loads = rng.integers(0, 60, size=n)
    chunk = rng.integers(0, n_chunks, size=n)
    bin_of, off, items, bl = SA.sa_lpt_schedule_grouped(loads, chunk, n_chunks, n_groups, n_groups * per)
    cl = np.bincount(chunk, weights=loads, minlength=n_chunks).astype(np.int64)
    g_of_chunk = O.lpt_schedule(cl.tolist(), n_groups)[0]
    for g in range(n_groups):
        mem = np.flatnonzero(np.asarray(g_of_chunk)[chunk] == g)
        rb, roff, ritems, rload = O.lpt_schedule(loads[mem].tolist(), per)
        for lb in range(per):
            gb = lb * n_groups + g
            assert items[off[gb]:off[gb + 1]].tolist() == mem[ritems[roff[lb]:roff[lb + 1]]].tolist()
            assert int(bl[gb]) == int(rload[lb])
    assert np.all(bin_of[items] == np.repeat(np.arange(n_groups * per), np.diff(off)))
    with pytest.raises(SA.SaError):
        SA.sa_lpt_schedule_grouped(loads, chunk, n_chunks, 3, 7)


def test_lpt_on_config_tile_loads():
    """The tile loads of the 32K Llama-shaped workload scheduled onto 512 bins:
    identical to the oracle, and the makespan within one item of the mean."""
    spec = W.LLAMA_32K
    bud = W.prefill_budgets(spec, W.seed_of(W.LLAMA_32K))
    import torch
    q = torch.empty((1, spec.n_q_heads, spec.seq_len, spec.head_dim), dtype=torch.bfloat16, device="meta")
    k = torch.empty((1, spec.n_kv_heads, spec.seq_len, spec.head_dim), dtype=torch.bfloat16, device="meta")
    desc = SA.make_prefill_desc(q, k, k, q, spec.block)
    counts, kmax = SA.sa_prefill_block_counts(desc, SA.make_budgets(bud))
    loads = counts.reshape(-1)
    got = SA.sa_lpt_schedule(loads, 512)
    ref = O.lpt_schedule(loads.tolist(), 512)
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)
    assert got[3].max() <= loads.sum() / 512 + loads.max()


def test_block_counts_match_budget_rule():
    import torch
    for spec, seed in ((W.TINY_F32, 1000), (W.LLAMA_128K.with_(seq_len=8192 + 64), 7), (W.QWEN_64K, 1003)):
        bud = W.prefill_budgets(spec, seed)
        q = torch.empty((1, spec.n_q_heads, spec.seq_len, spec.head_dim), device="meta",
                        dtype=torch.float32 if spec.dtype == "f32" else torch.bfloat16)
        k = torch.empty((1, spec.n_kv_heads, spec.seq_len, spec.head_dim), device="meta", dtype=q.dtype)
        desc = SA.make_prefill_desc(q, k, k, q, spec.block)
        counts, kmax = SA.sa_prefill_block_counts(desc, SA.make_budgets(bud))
        for h in range(spec.n_q_heads):
            ref = [O.budget_blocks(m + 1, bud["min_blocks"][h], bud["ratio_q16"][h]) for m in range(spec.n_blocks)]
            assert counts[0, h].tolist() == ref
        assert kmax == counts.max()
    dspec = W.DECODE_128K
    bud = W.decode_budgets(dspec, 1004)
    q = torch.empty((dspec.batch, dspec.n_q_heads, dspec.head_dim), dtype=torch.bfloat16, device="meta")
    k = torch.empty((dspec.batch, dspec.n_kv_heads, dspec.kv_len, dspec.head_dim), dtype=torch.bfloat16,
                    device="meta")
    desc = SA.make_decode_desc(q, k, k, q)
    counts, kmax = SA.sa_decode_block_counts(desc, SA.make_budgets(bud))
    for h in range(dspec.n_q_heads):
        nc = -(-dspec.kv_len // int(bud["granularity"][h]))
        assert counts[h] == O.budget_blocks(nc, bud["min_blocks"][h], bud["ratio_q16"][h])


def _desc(**kw):
    import torch
    q = torch.empty((1, 4, 1024, 64), dtype=torch.bfloat16, device="meta")
    k = torch.empty((1, 2, 1024, 64), dtype=torch.bfloat16, device="meta")
    d = SA.make_prefill_desc(q, k, k, q, 64)
    for key, val in kw.items():
        setattr(d, key, val)
    return d


def _bud(**kw):
    b = {"min_blocks": [2] * 4, "ratio_q16": [4096] * 4, "n_sink": [1] * 4, "n_local": [1] * 4,
         "granularity": [64] * 4}
    b.update(kw)
    return SA.make_budgets(b)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), SA.SA_ERR_UNSUPPORTED),
    (dict(n_kv_heads=3), SA.SA_ERR_INVALID_ARG),
    (dict(block_size=32), SA.SA_ERR_UNSUPPORTED),
    (dict(kv_len=512), SA.SA_ERR_INVALID_ARG),
    (dict(dtype=7), SA.SA_ERR_INVALID_ARG),
    (dict(kernel_variant=3), SA.SA_ERR_INVALID_ARG),
    (dict(batch=0), SA.SA_ERR_INVALID_ARG),
])
def test_invalid_descriptors_rejected(kw, code):
    with pytest.raises(SA.SaError) as e:
        SA.sa_prefill_block_counts(_desc(**kw), _bud())
    assert e.value.status == code


@pytest.mark.parametrize("kw", [dict(min_blocks=[1] * 4), dict(n_sink=[-1] * 4), dict(ratio_q16=[70000] * 4),
                                dict(min_blocks=[0] * 4, n_sink=[0] * 4, n_local=[0] * 4)])
def test_invalid_budgets_rejected(kw):
    with pytest.raises(SA.SaError) as e:
        SA.sa_prefill_block_counts(_desc(), _bud(**kw))
    assert e.value.status == SA.SA_ERR_INVALID_ARG


def test_slices_beyond_32_bit_offsets_rejected():
    """A (sequence, KV head) slice of K or V at or beyond 2 GiB would overflow the
    kernels' 32-bit buffer offsets: rejected before any launch."""
    import torch
    L = 1 << 16
    q = torch.empty((1, 4, L, 128), dtype=torch.bfloat16, device="meta")
    # rows 64 KiB apart (a wide packed-projection buffer): 2^16 rows span 4 GiB
    k = torch.empty_strided((1, 2, L, 128), (2 * L * 32768, 32768, 32768, 1), dtype=torch.bfloat16,
                            device="meta")
    d = SA.make_prefill_desc(q, k, k, q, 128)
    b = SA.make_budgets({"min_blocks": [2] * 4, "ratio_q16": [0] * 4, "n_sink": [1] * 4, "n_local": [1] * 4,
                         "granularity": [128] * 4})
    fake = ctypes.c_void_p(1 << 20)
    st = SA._lib.sa_sparse_attn_prefill(ctypes.byref(d), fake, fake, fake, fake, None, fake, fake, 2, None, None, None,
                                        0, 0, None, 0, None)
    assert st == SA.SA_ERR_UNSUPPORTED and "2 GiB" in SA._lib.sa_last_error().decode()
    qd = torch.empty((1, 4, 128), dtype=torch.bfloat16, device="meta")
    kd = torch.empty_strided((1, 1, L, 128), (L * 32768, L * 32768, 32768, 1), dtype=torch.bfloat16,
                             device="meta")
    dd = SA.make_decode_desc(qd, kd, kd, qd)
    bd = SA.make_budgets({"min_blocks": [2] * 4, "ratio_q16": [0] * 4, "n_sink": [1] * 4, "n_local": [1] * 4,
                          "granularity": [64] * 4})
    st = SA._lib.sa_sparse_attn_decode(ctypes.byref(dd), bd, fake, fake, fake, fake, None, fake, fake, 2, 0, fake,
                                       1 << 40, None)
    assert st == SA.SA_ERR_UNSUPPORTED and "2 GiB" in SA._lib.sa_last_error().decode()


def test_device_calls_fail_cleanly_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = _desc()
    b = _bud()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation and the device check come first
    lib = SA._lib
    st = lib.sa_select_blocks(ctypes.byref(d), b, fake, fake, None, fake, fake, 64, None, fake, 1 << 30, None)
    assert st in (SA.SA_ERR_NO_DEVICE, SA.SA_ERR_HIP)
    st = lib.sa_select_blocks(ctypes.byref(d), b, fake, fake, None, fake, fake, 1, None, fake, 1 << 30, None)
    assert st == SA.SA_ERR_INVALID_ARG  # kmax below the largest count, caught before the device check
    st = lib.sa_select_blocks(ctypes.byref(d), b, fake, fake, None, fake, fake, 64, None, fake, 16, None)
    assert st == SA.SA_ERR_WORKSPACE
    st = lib.sa_select_blocks(ctypes.byref(d), b, fake, fake, None, fake, fake, 64, ctypes.c_void_p((1 << 20) + 2),
                              fake, 1 << 30, None)
    assert st == SA.SA_ERR_INVALID_ARG  # misaligned key_norms
    st = lib.sa_sparse_attn_prefill(ctypes.byref(d), fake, fake, fake, fake, None, fake, fake, 16, None, None, None, 0,
                                    0, None, 0, None)
    assert st in (SA.SA_ERR_NO_DEVICE, SA.SA_ERR_HIP)
    st = lib.sa_sparse_attn_prefill(ctypes.byref(d), ctypes.c_void_p(3), fake, fake, fake, None, fake, fake, 16,
                                    None, None, None, 0, 0, None, 0, None)
    assert st == SA.SA_ERR_INVALID_ARG  # misaligned q
    st = lib.sa_sparse_attn_prefill(ctypes.byref(d), fake, fake, fake, fake, None, fake, fake, 16,
                                    ctypes.c_void_p((1 << 20) + 2), None, None, 0, 0, None, 0, None)
    assert st == SA.SA_ERR_INVALID_ARG  # misaligned key_norms


def _paged_call(page_size=128, max_pages=8, pages_per_head=20, dtype="bf16", table=True, pages_null=False,
                L=1000):
    """Return the status of sa_sparse_attn_decode_paged on fake device pointers."""
    import torch
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd = torch.empty((2, 4, 128), dtype=dt, device="meta")
    kp = torch.empty((2, 4, 128, 128), dtype=dt, device="meta")  # the pool shape only sets the strides
    d = SA.make_paged_decode_desc(qd, kp, kp, L)
    b = SA.make_budgets({"min_blocks": [2] * 4, "ratio_q16": [0] * 4, "n_sink": [1] * 4, "n_local": [1] * 4,
                        "granularity": [64] * 4})
    pg = SA.sa_kv_pages()
    pg.table = (1 << 20) if table else None
    pg.page_size, pg.max_pages, pg.pages_per_head = page_size, max_pages, pages_per_head
    fake = ctypes.c_void_p(1 << 20)
    st = SA._lib.sa_sparse_attn_decode_paged(ctypes.byref(d), b, fake, fake, fake,
                                             None if pages_null else ctypes.byref(pg), fake, None, fake, fake, 2, 0,
                                             fake, 1 << 40, None)
    _paged_call.last_error = SA._lib.sa_last_error().decode()
    st2 = SA._lib.sa_pool_keys_decode_paged(ctypes.byref(d), b, fake, None if pages_null else ctypes.byref(pg),
                                            fake, None)
    return st, st2


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=96), SA.SA_ERR_INVALID_ARG),       # not a multiple of 64
    (dict(page_size=0), SA.SA_ERR_INVALID_ARG),
    (dict(max_pages=7), SA.SA_ERR_INVALID_ARG),        # 7 pages of 128 < 1000 tokens
    (dict(pages_per_head=0), SA.SA_ERR_INVALID_ARG),
    (dict(table=False), SA.SA_ERR_INVALID_ARG),
    (dict(pages_null=True), SA.SA_ERR_INVALID_ARG),
    (dict(page_size=1 << 16, max_pages=1, pages_per_head=1 << 8), SA.SA_ERR_UNSUPPORTED),  # pool of 4 GiB
])
def test_paged_arguments_rejected(kw, code):
    st, st2 = _paged_call(**kw)
    assert st == code, _paged_call.last_error
    assert st2 == code


def test_paged_decode_fp32_unsupported_and_valid_call_reaches_device_check():
    import torch
    st, st2 = _paged_call(dtype="f32")
    assert st == SA.SA_ERR_UNSUPPORTED and "bf16" in _paged_call.last_error
    st, st2 = _paged_call()
    if not torch.cuda.is_available():
        assert st in (SA.SA_ERR_NO_DEVICE, SA.SA_ERR_HIP) and st2 in (SA.SA_ERR_NO_DEVICE, SA.SA_ERR_HIP)


def test_paged_pool_builder_scatters_exactly():
    """The seeded page pools hold every cache row at the page the table names,
    zero rows past the cache end, and a permutation of pages per KV head."""
    import torch
    spec = W.DECODE_128K.with_(batch=2, kv_len=1000)
    inp = W.make_decode(spec, 3)
    pk = W.make_paged(inp.k, inp.v, 128, 5)
    b, hk, L, D = inp.k.shape
    tab = pk.table.numpy()
    for j in range(hk):
        flat = tab[:, j].reshape(-1)
        assert len(set(flat.tolist())) == flat.size and flat.min() >= 0 and flat.max() < pk.k_pages.shape[1]
    back_k = torch.stack([torch.stack([pk.k_pages[j, torch.from_numpy(tab[bi, j]).long()].reshape(-1, D)[:L]
                                       for j in range(hk)]) for bi in range(b)])
    back_v = torch.stack([torch.stack([pk.v_pages[j, torch.from_numpy(tab[bi, j]).long()].reshape(-1, D)[:L]
                                       for j in range(hk)]) for bi in range(b)])
    assert torch.equal(back_k, inp.k) and torch.equal(back_v, inp.v)
    last = pk.k_pages[0, int(tab[0, 0, -1])]
    assert torch.count_nonzero(last[L % 128:]) == 0


@pytest.mark.parametrize("seed", range(4))
def test_lpt_queue_order_tiered(seed):
    """Tiers floor(t log2 k) exact in integers (bit length of k^t, minus one),
    heaviest tier first, then group, then load, then index: against a plain
    sort with the same key."""
    r = np.random.default_rng(seed)
    n = 700
    loads = r.integers(0, 300, n)
    loads[:5] = [1, 2, 4, 8, 0]  # exact powers of two sit at tier boundaries
    groups = r.integers(0, 6, n).astype(np.int32)
    for t in (1, 2, 4):
        tier = [int(max(int(x), 1) ** t).bit_length() - 1 for x in loads]
        want = sorted(range(n), key=lambda i: (-tier[i], int(groups[i]), -int(loads[i]), i))
        assert SA.sa_lpt_queue_order_tiered(loads, groups, t).tolist() == want
    want = sorted(range(n), key=lambda i: (-(int(max(int(loads[i]), 1) ** 4).bit_length() - 1), -int(loads[i]), i))
    assert SA.sa_lpt_queue_order_tiered(loads, None, 4).tolist() == want
    with pytest.raises(SA.SaError):
        SA.sa_lpt_queue_order_tiered(loads, groups, 3)
    with pytest.raises(SA.SaError):
        SA.sa_lpt_queue_order_tiered(np.array([1 << 15]), None, 4)


@pytest.mark.parametrize("seed", range(6))
def test_lpt_queue_partition(seed):
    """Partitioned queue: the tiered order (tier, group, load, index) cut into
    runs of one (tier, group) of at most chunk items, the runs placed by the
    oracle's greedy LPT on their loads, each partition keeping the tiered order,
    partitions concatenated with their offsets."""
    r = np.random.default_rng(200 + seed)
    n_groups = int(r.integers(1, 20))
    n_queues = int(r.integers(1, 17))
    chunk = [1, 3, 64, 0][seed % 4]
    n = int(r.integers(0, 900))
    loads = r.integers(0, 300, n)
    groups = r.integers(0, n_groups, n).astype(np.int32)
    order, off = SA.sa_lpt_queue_partition(loads, groups, n_groups, n_queues, 4, chunk)
    chunk = chunk or n + 1  # 0: no limit
    tier = [int(max(int(x), 1) ** 4).bit_length() - 1 for x in loads]
    seq = sorted(range(n), key=lambda i: (-tier[i], int(groups[i]), -int(loads[i]), i))
    units, unit_load = [], []
    for p, i in enumerate(seq):
        prev = seq[p - 1] if p else None
        if prev is None or (tier[prev], groups[prev]) != (tier[i], groups[i]) or len(units[-1]) == chunk:
            units.append([])
            unit_load.append(0)
        units[-1].append(i)
        unit_load[-1] += int(loads[i])
    q_of_u, _, _, _ = O.lpt_schedule(unit_load, n_queues) if units else ([], None, None, None)
    rank = {i: p for p, i in enumerate(seq)}
    want, want_off = [], [0]
    for qq in range(n_queues):
        want += sorted((i for u, items in enumerate(units) if q_of_u[u] == qq for i in items), key=rank.get)
        want_off.append(len(want))
    assert order.tolist() == want and off.tolist() == want_off
    with pytest.raises(SA.SaError):
        SA.sa_lpt_queue_partition(loads, groups, n_groups, 17)
    with pytest.raises(SA.SaError):
        SA.sa_lpt_queue_partition(loads, groups, n_groups, n_queues, 4, -1)
    if n:
        bad = groups.copy()
        bad[0] = n_groups
        with pytest.raises(SA.SaError):
            SA.sa_lpt_queue_partition(loads, bad, n_groups, n_queues)


def test_prefill_queues_validation():
    """The partitioned prefill queue rejects bad partitions before any launch;
    valid ones reach the device check."""
    import torch
    d = _desc()
    fake = ctypes.c_void_p(1 << 20)
    lib = SA._lib
    counts, _ = SA.sa_prefill_block_counts(d, _bud())
    tiles = counts.size

    def call(off, nq=None, nwg=8, ws=256):
        a = np.ascontiguousarray(off, dtype=np.int32)
        return lib.sa_sparse_attn_prefill_queues(ctypes.byref(d), fake, fake, fake, fake, None, fake, fake, 16, None,
                                                 a.ctypes.data_as(SA._i32p), a.size - 1 if nq is None else nq,
                                                 fake, nwg, 0, fake, ws, None)

    assert call([0, tiles // 2, tiles + 1]) == SA.SA_ERR_INVALID_ARG  # does not end at the tile count
    assert call([1, tiles]) == SA.SA_ERR_INVALID_ARG                  # does not start at 0
    assert call([0, tiles // 2 + 1, tiles // 2, tiles]) == SA.SA_ERR_INVALID_ARG  # decreasing
    assert call([0] * 18 + [tiles]) == SA.SA_ERR_INVALID_ARG          # 18 partitions
    assert call([0, tiles], nwg=0) == SA.SA_ERR_INVALID_ARG
    assert call([0, 3, tiles], ws=4) == SA.SA_ERR_INVALID_ARG         # 2 counters need 8 bytes
    if not torch.cuda.is_available():
        assert call([0, 3, tiles]) in (SA.SA_ERR_NO_DEVICE, SA.SA_ERR_HIP)


def test_output_deviation_validation():
    """sa_output_deviation rejects NULL and misaligned pointers before any
    launch; valid ones reach the device check."""
    import torch
    d = _desc()
    lib = SA._lib
    fake = ctypes.c_void_p(1 << 20)
    assert lib.sa_output_deviation(ctypes.byref(d), None, fake, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_output_deviation(ctypes.byref(d), ctypes.c_void_p((1 << 20) + 4), fake, fake,
                                   None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_output_deviation(ctypes.byref(d), fake, fake, ctypes.c_void_p((1 << 20) + 4),
                                   None) == SA.SA_ERR_INVALID_ARG
    if not torch.cuda.is_available():
        assert lib.sa_output_deviation(ctypes.byref(d), fake, fake, fake, None) in (SA.SA_ERR_NO_DEVICE,
                                                                                     SA.SA_ERR_HIP)


def test_measure_probes_validation():
    """The rate probes reject bad sizes and pointers before any launch; valid
    calls reach the device check."""
    import torch
    lib = SA._lib
    fake = ctypes.c_void_p(1 << 20)
    assert lib.sa_measure_mfma_peak(0, 16, 0, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_mfma_peak(256, 0, 0, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_mfma_peak(256, 65537, 1, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_mfma_peak(256, 16, 2, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_mfma_peak(256, 16, -1, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_mfma_peak(256, 16, 0, None, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_mfma_peak(256, 16, 0, ctypes.c_void_p((1 << 20) + 2), None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_hbm_read(fake, 100, 256, fake, None) == SA.SA_ERR_INVALID_ARG   # not a multiple of 16
    assert lib.sa_measure_hbm_read(fake, 0, 256, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_hbm_read(ctypes.c_void_p((1 << 20) + 8), 1 << 20, 256, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_hbm_read(fake, 1 << 20, 0, fake, None) == SA.SA_ERR_INVALID_ARG
    assert lib.sa_measure_hbm_read(None, 1 << 20, 256, fake, None) == SA.SA_ERR_INVALID_ARG
    if not torch.cuda.is_available():
        assert lib.sa_measure_mfma_peak(256, 16, 1, fake, None) in (SA.SA_ERR_NO_DEVICE, SA.SA_ERR_HIP)
        assert lib.sa_measure_hbm_read(fake, 1 << 20, 256, fake, None) in (SA.SA_ERR_NO_DEVICE, SA.SA_ERR_HIP)


def _sched_case(seed):
    """A batch-2, 8-query-head, 2-KV-head prefill descriptor with per-head
    budgets, its tile loads (the oracle's budget rule) and group keys."""
    import torch
    rng = np.random.default_rng(seed)
    S, Hq, Hkv, blk = 64 * 37, 8, 2, 64
    q = torch.empty((2, Hq, S, 64), dtype=torch.bfloat16, device="meta")
    k = torch.empty((2, Hkv, S, 64), dtype=torch.bfloat16, device="meta")
    d = SA.make_prefill_desc(q, k, k, q, blk)
    bud = {"min_blocks": [2] * Hq, "ratio_q16": [int(x) for x in rng.integers(1000, 40000, Hq)],
           "n_sink": [1] * Hq, "n_local": [1] * Hq, "granularity": [blk] * Hq}
    nb = -(-S // blk)
    loads = np.array([O.budget_blocks(m + 1, 2, bud["ratio_q16"][h]) for b in range(2) for h in range(Hq)
                      for m in range(nb)], dtype=np.int64)
    bh = np.arange(loads.size) // nb
    return d, SA.make_budgets(bud), loads, bh, nb, Hq, Hkv


@pytest.mark.parametrize("seed", [0, 1])
def test_prefill_schedule_bins(seed):
    """sa_prefill_schedule's bins are the greedy placement of the budget rule's
    tile loads (the oracle's LPT), walked in item or assignment order, and the
    two-level form equals sa_lpt_schedule_grouped on (sequence, KV head, chunk)
    keys written out here from their definition."""
    d, b, loads, bh, nb, Hq, Hkv = _sched_case(seed)
    for n_bins in (1, 7, 64):
        items, off, load = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_BINS, n_bins=n_bins, bin_order=1)
        _, w_off, w_items, w_load = O.lpt_schedule(loads.tolist(), n_bins)
        assert load.tolist() == w_load.tolist()
        assert off.tolist() == w_off.tolist() and items.tolist() == w_items.tolist()
        items0, off0, _ = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_BINS, n_bins=n_bins, bin_order=0)
        assert off0.tolist() == off.tolist()
        for bn in range(n_bins):
            assert items0[off[bn]:off[bn + 1]].tolist() == sorted(items[off[bn]:off[bn + 1]].tolist())
    G = Hq // Hkv
    chunk_len = 8
    n_m = -(-nb // chunk_len)
    it = np.arange(loads.size)
    bb, hh, mm = bh // Hq, bh % Hq, it % nb
    chunk = ((bb * Hkv + hh // G) * n_m + mm // chunk_len).astype(np.int32)
    _, off_w, items_w, load_w = SA.sa_lpt_schedule_grouped(loads, chunk, int(chunk.max()) + 1, 4, 16)
    items, off, load = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_BINS_XCD, n_bins=16, bin_order=1, xcd_groups=4,
                                              xcd_chunk=chunk_len)
    assert items.tolist() == items_w.tolist() and off.tolist() == off_w.tolist() and load.tolist() == load_w.tolist()


@pytest.mark.parametrize("seed", [0, 1])
def test_prefill_schedule_queue(seed):
    """The queue orders: KV-tier order and partitions equal the calls they
    name on (sequence, KV head) keys; the "head" order puts heads in
    non-increasing total load, each head's tiles together, longest first."""
    d, b, loads, bh, nb, Hq, Hkv = _sched_case(seed)
    G = Hq // Hkv
    kv = (bh // G).astype(np.int32)
    items, off, load = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_QUEUE, queue_group=0, n_queues=1)
    assert load is None and off.tolist() == [0, loads.size]
    assert items.tolist() == SA.sa_lpt_queue_order_tiered(loads, kv, 4).tolist()
    items, off, _ = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_QUEUE, queue_group=0, n_queues=8, queue_chunk=5)
    w_items, w_off = SA.sa_lpt_queue_partition(loads, kv, 2 * Hkv, 8, 4, 5)
    assert items.tolist() == w_items.tolist() and off.tolist() == w_off.tolist()
    items, _, _ = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_QUEUE, queue_group=1)
    assert items.tolist() == SA.sa_lpt_queue_order(loads, kv).tolist()
    items, _, _ = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_QUEUE, queue_group=3)
    assert items.tolist() == SA.sa_lpt_queue_order(loads, None).tolist()
    items, _, _ = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_QUEUE, queue_group=2)
    heads = bh[items]
    tot = np.bincount(bh, weights=loads)
    runs = [heads[0]] + [heads[i] for i in range(1, heads.size) if heads[i] != heads[i - 1]]
    assert len(runs) == tot.size  # each head's tiles are contiguous
    assert all(tot[runs[i]] >= tot[runs[i + 1]] for i in range(len(runs) - 1))
    for h in runs:
        seg = loads[items[heads == h]]
        assert np.all(seg[:-1] >= seg[1:])


def test_prefill_schedule_auto():
    """SA_QUEUE_AUTO: up to 256 query blocks per head, plain longest first on
    one queue; beyond, the tiered order in n_queues partitions."""
    import torch
    d, b, loads, bh, nb, Hq, Hkv = _sched_case(0)  # 37 query blocks
    items, off, _ = SA.sa_prefill_schedule(d, b, SA.SA_SCHED_QUEUE, queue_group=SA.QUEUE_GROUPS["auto"], n_queues=8)
    assert off.tolist() == [0, loads.size]
    assert items.tolist() == SA.sa_lpt_queue_order(loads, None).tolist()
    rng = np.random.default_rng(5)
    for S, want_parts in ((256 * 64, False), (257 * 64, True), (300 * 64 + 5, True)):
        q = torch.empty((1, 4, S, 64), dtype=torch.bfloat16, device="meta")
        k = torch.empty((1, 2, S, 64), dtype=torch.bfloat16, device="meta")
        dd = SA.make_prefill_desc(q, k, k, q, 64)
        bud = {"min_blocks": [2] * 4, "ratio_q16": [int(x) for x in rng.integers(1000, 40000, 4)],
               "n_sink": [1] * 4, "n_local": [1] * 4, "granularity": [64] * 4}
        bb = SA.make_budgets(bud)
        n_b = -(-S // 64)
        ld = np.array([O.budget_blocks(m + 1, 2, bud["ratio_q16"][h]) for h in range(4) for m in range(n_b)],
                      dtype=np.int64)
        items, off, _ = SA.sa_prefill_schedule(dd, bb, SA.SA_SCHED_QUEUE, queue_group=SA.QUEUE_GROUPS["auto"],
                                               n_queues=8)
        if want_parts:
            kv = (np.arange(ld.size) // n_b // 2).astype(np.int32)
            w_items, w_off = SA.sa_lpt_queue_partition(ld, kv, 2, 8, 4, 0)
            assert items.tolist() == w_items.tolist() and off.tolist() == w_off.tolist()
        else:
            assert off.tolist() == [0, ld.size]
            assert items.tolist() == SA.sa_lpt_queue_order(ld, None).tolist()


def test_prefill_schedule_validation():
    d, b, *_ = _sched_case(0)
    for kw in (dict(kind=9), dict(kind=SA.SA_SCHED_BINS, n_bins=0), dict(kind=SA.SA_SCHED_BINS_XCD, n_bins=6,
                                                                         xcd_groups=4, xcd_chunk=8),
               dict(kind=SA.SA_SCHED_BINS, n_bins=4, bin_order=2), dict(kind=SA.SA_SCHED_QUEUE, queue_group=7),
               dict(kind=SA.SA_SCHED_QUEUE, queue_group=1, n_queues=4),
               dict(kind=SA.SA_SCHED_QUEUE, queue_group=0, n_queues=17)):
        with pytest.raises(SA.SaError):
            SA.sa_prefill_schedule(d, b, **kw)
    assert SA.sa_prefill_schedule(d, b, SA.SA_SCHED_GRID) == (None, None, None)


def test_prefill_selection_block_limit():
    """The prefill selection holds a workgroup's score rows in LDS: more than
    8192 query blocks is SA_ERR_UNSUPPORTED, found before any device call."""
    import torch
    q = torch.empty((1, 1, 8193 * 64, 64), dtype=torch.bfloat16, device="meta")
    d = SA.make_prefill_desc(q, q, q, q, 64)
    b = SA.make_budgets({"min_blocks": [2], "ratio_q16": [4096], "n_sink": [1], "n_local": [1], "granularity": [64]})
    with pytest.raises(SA.SaError) as e:
        SA.sa_prefill_block_counts(d, b)
    assert e.value.status == SA.SA_ERR_UNSUPPORTED
    fake = ctypes.c_void_p(1 << 20)
    st = SA._lib.sa_select_blocks(ctypes.byref(d), b, fake, fake, None, fake, fake, 8193, None, fake, 1 << 40, None)
    assert st == SA.SA_ERR_UNSUPPORTED
    q8 = q[:, :, : 8192 * 64]
    d8 = SA.make_prefill_desc(q8, q8, q8, q8, 64)
    _, kmax8 = SA.sa_prefill_block_counts(d8, b)
    st = SA._lib.sa_select_blocks(ctypes.byref(d8), b, fake, fake, None, fake, fake, kmax8, None, fake, 1 << 40, None)
    if not torch.cuda.is_available():
        assert st in (SA.SA_ERR_NO_DEVICE, SA.SA_ERR_HIP)
