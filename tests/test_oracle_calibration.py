"""Pins of the calibration oracle (block attention mass, head recovery, max-min
budget shifting).  They need no built library: the host library's calibration
is checked against this oracle in test_abi_calibration.py.

Mass: every row of softmax probabilities sums to one, so row m of the block
mass sums to the query rows of block m; with Q = 0 every visible key of row t
has probability 1/(t+1), a closed form; and the block sums of
torch's fp64 softmax agree.  Recovery: a full budget keeps everything, a budget
of the forced blocks keeps exactly them, and the best selection is the best of
all block subsets.  Shifting: on tables that grow with the ratio, the lowest
recovery it reaches is the largest that any allocation of the total reaches.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O

def _qk(seed, b=1, H=2, Hk=1, S=300, D=16, scale=1.0):
    r = np.random.default_rng(seed)
    q = (scale * r.standard_normal((b, H, S, D))).astype(np.float32)
    k = (scale * r.standard_normal((b, Hk, S, D))).astype(np.float32)
    return q, k


def test_mass_rows_sum_to_row_count():
    q, k = _qk(1, S=300)
    W = O.block_attention_mass(q, k, 64)
    rows = np.array([min(64, 300 - 64 * m) for m in range(5)], dtype=np.float64)
    np.testing.assert_allclose(W.sum(axis=3), np.broadcast_to(rows, W.shape[:3]), rtol=0, atol=1e-12)
    assert np.all(np.triu(W[0, 0], 1) == 0)


def test_mass_uniform_attention_closed_form():
    q, k = _qk(2, S=200)
    q[:] = 0.0
    W = O.block_attention_mass(q, k, 32)
    nb = 7
    for m in range(nb):
        for n in range(m + 1):
            want = 0.0
            for t in range(32 * m, min(200, 32 * m + 32)):
                seen = max(0, min(t, 32 * n + 31) - 32 * n + 1)
                want += seen / (t + 1)
            assert abs(W[0, 0, m, n] - want) < 1e-12


def test_mass_matches_torch_softmax_block_sums():
    q, k = _qk(3, H=4, Hk=2, S=256, D=32)
    W = O.block_attention_mass(q, k, 64)
    qt, kt = torch.from_numpy(q).double(), torch.from_numpy(k).double()
    z = qt @ kt.repeat_interleave(2, dim=1).transpose(-1, -2) / math.sqrt(32)
    z = z.masked_fill(~torch.tril(torch.ones(256, 256, dtype=torch.bool)), float("-inf"))
    p = torch.softmax(z, dim=-1).numpy()
    ref = p.reshape(1, 4, 4, 64, 4, 64).sum(axis=(3, 5))
    np.testing.assert_allclose(W, ref, rtol=0, atol=1e-12)


def test_recovery_full_budget_and_forced_only():
    q, k = _qk(4, S=320, scale=2.0)
    W = O.block_attention_mass(q, k, 64)
    assert O.head_recovery(W[:, 0], 65536, 2, 1, 1) == 1.0
    got = O.head_recovery(W[:, 0], 1, 2, 1, 1)  # tiny ratio: only the sink and the diagonal
    want = np.mean([1.0] + [(W[0, 0, m, 0] + W[0, 0, m, m]) / W[0, 0, m, :m + 1].sum() for m in range(1, 5)])
    assert abs(got - want) < 1e-14


def test_row_recovery_is_the_best_subset():
    r = np.random.default_rng(5)
    for trial in range(30):
        n = int(r.integers(3, 9))
        w = r.random(n) ** 3
        if trial % 5 == 0:
            w[r.integers(0, n, 2)] = w[0]  # ties
        for kk in range(2, n + 1):
            best = 0.0
            for sub in itertools.combinations(range(1, n - 1), kk - 2):
                best = max(best, w[0] + w[n - 1] + sum(w[list(sub)]))
            assert abs(O.row_recovery(w, kk, 1, 1) * w.sum() - best) < 1e-12


def _monotone_tables(seed, H, n_grid):
    r = np.random.default_rng(seed)
    steps = r.random((H, n_grid)) * (r.random((H, n_grid)) < 0.7)
    rec = np.cumsum(steps, axis=1)
    return rec / rec[:, -1:].clip(min=1e-9) * r.uniform(0.8, 1.0, (H, 1))


@pytest.mark.parametrize("seed", range(8))
def test_maxmin_shift_reaches_the_brute_force_optimum(seed):
    H, n_grid, step = 3 + seed % 2, 8, 8192
    rec = _monotone_tables(seed, H, n_grid)
    for per_units in (1, 2, 4):
        total = H * per_units * step
        got = O.maxmin_shift(rec, total, step)
        assert sum(got) == total and all(step <= x <= 65536 for x in got)
        got_min = min(rec[h, got[h] // step - 1] for h in range(H))
        assert got_min == O.brute_force_maxmin(rec, total, step)
        assert got_min >= rec[:, per_units - 1].min()  # never below the equal split


def test_needed_ratio():
    rec = np.array([0.2, 0.5, 0.89, 0.9, 0.95])
    assert O.needed_ratio(rec, 0.9, 4096) == 4 * 4096
    assert O.needed_ratio(rec, 0.99, 4096) == 5 * 4096


def _budget(H, min_blocks=2):
    return {"min_blocks": [min_blocks] * H, "ratio_q16": [0] * H, "n_sink": [1] * H, "n_local": [1] * H}


# ---------------------------------------------------------------- output deviation (R37)


def _dev_budget(H, ratio, block):
    return {"min_blocks": [2] * H, "ratio_q16": [ratio] * H, "n_sink": [1] * H, "n_local": [1] * H,
            "granularity": [block] * H}


def _qkv(seed, b=2, H=4, Hk=2, S=512, D=16):
    r = np.random.default_rng(seed)
    q = r.standard_normal((b, H, S, D)).astype(np.float32)
    k = r.standard_normal((b, Hk, S, D)).astype(np.float32)
    v = r.standard_normal((b, Hk, S, D)).astype(np.float32)
    return q, k, v


def test_output_deviation_hand_values():
    """Relative Frobenius distance, pooled over sequences: one sequence 4/3;
    two sequences (differences 4 and 0, reference norms 3 and 4) 4/5, not the
    mean of 4/3 and 0."""
    a = np.array([[[[3.0, 4.0]]]])
    r = np.array([[[[3.0, 0.0]]]])
    assert O.output_deviation(a, r)[0] == pytest.approx(4.0 / 3.0, abs=1e-15)
    a2 = np.array([[[[3.0, 4.0]]], [[[0.0, 4.0]]]])
    r2 = np.array([[[[3.0, 0.0]]], [[[0.0, 4.0]]]])
    assert O.output_deviation(a2, r2)[0] == pytest.approx(0.8, abs=1e-15)
    assert O.needed_ratio_deviation([0.5, 0.2, 0.05, 0.01], 0.1, 4096) == 3 * 4096
    assert O.needed_ratio_deviation([0.5, 0.2], 0.01, 4096) == 2 * 4096


def test_output_deviation_split_identity():
    """Dense attention splits over the kept and the dropped keys: with w the
    dropped keys' softmax weight (from the two log-sum-exps),
    o_dense = (1 - w) o_kept + w o_dropped, so o_dense - o_kept = w (o_dropped -
    o_kept).  The deviation the table reports must equal the one built from
    this split, computed from separate softmaxes over disjoint key sets."""
    q, k, v = _qkv(11)
    block, step = 64, 16384
    dev = O.deviation_table(q, k, v, _dev_budget(4, 0, block), block, step)
    assert dev.shape == (4, 4)
    nb = 512 // block
    for i in range(4):
        ratio = (i + 1) * step
        idx, cnt = O.select_blocks_prefill(q, k, _dev_budget(4, ratio, block), block)
        o_kept, l_kept = O.attention_prefill_gather(q, k, v, idx, cnt, block)
        # the dropped causal blocks of every tile
        comp = np.full((2, 4, nb, nb), -1, dtype=np.int32)
        ccnt = np.zeros((2, 4, nb), dtype=np.int32)
        for bi in range(2):
            for h in range(4):
                for m in range(nb):
                    rest = sorted(set(range(m + 1)) - set(idx[bi, h, m, :cnt[bi, h, m]].tolist()))
                    comp[bi, h, m, :len(rest)] = rest
                    ccnt[bi, h, m] = len(rest)
        some = [(bi, h, m) for bi in range(2) for h in range(4) for m in range(nb) if ccnt[bi, h, m]]
        o_out, l_out = O.attention_prefill_gather(q, k, v, comp, ccnt, block, tiles=some)
        o_out = np.nan_to_num(o_out)  # tiles with nothing dropped (left NaN): weight 0
        with np.errstate(invalid="ignore"):
            w = np.where(np.isfinite(l_out), 1.0 / (1.0 + np.exp(l_kept - l_out)), 0.0)[..., None]
        diff = w * (o_out - o_kept)
        dense = (1.0 - w) * o_kept + w * o_out
        want = [math.sqrt(np.sum(diff[:, h] ** 2)) / math.sqrt(np.sum(dense[:, h] ** 2)) for h in range(4)]
        np.testing.assert_allclose(dev[:, i], want, rtol=1e-10, atol=1e-14)
    assert np.all(dev[:, -1] == 0.0)  # ratio 1 keeps every block
    assert np.all(dev[:, 0] > 0.05)   # a quarter of the blocks moves the output


def test_output_deviation_zero_cases():
    """Constant values: every softmax average is that constant, so no budget
    moves the output; the full budget alone on random values: zero."""
    q, k, v = _qkv(12, b=1, H=2, Hk=1, S=256)
    v[:] = 0.75
    dev = O.deviation_table(q, k, v, _dev_budget(2, 0, 64), 64, 16384)
    assert np.all(np.abs(dev) < 1e-14)
    q, k, v = _qkv(13, b=1, H=2, Hk=1, S=256)
    dev1 = O.deviation_table(q, k, v, _dev_budget(2, 0, 64), 64, 65536)
    assert dev1.shape == (2, 1) and np.all(dev1 == 0.0)
