"""Pins for the oracle's greedy longest-load-first placement.

Against a hand-worked example (tests/golden/lpt_config0.txt), brute-force
optimal partitions on up to 10 items, Graham's worst-case bound for the greedy
rule, and the structure the tie rules force.
"""

import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    d = {"bins": {}}
    for line in open(os.path.join(GOLDEN, "lpt_config0.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "loads":
            d["loads"] = [int(x) for x in f[1:]]
        elif f[0] == "bin":
            d["bins"][int(f[1])] = ([int(x) for x in f[3:f.index("load")]], int(f[-1]))
        else:
            d[f[0]] = int(f[1])
    return d


def test_golden_config0_heads_on_two_bins():
    g = _golden()
    bin_of, off, items, load = O.lpt_schedule(g["loads"], g["n_bins"])
    for b, (its, ld) in g["bins"].items():
        assert items[off[b]:off[b + 1]].tolist() == its
        assert load[b] == ld
        for i in its:
            assert bin_of[i] == b
    assert load.max() == g["makespan"]
    assert O.brute_force_makespan(g["loads"], g["n_bins"]) == g["optimal_makespan"]


def _opt_at_most_two_per_bin(loads, m):
    """Best makespan over assignments with at most two items per bin."""
    import itertools
    n = len(loads)
    best = None
    for a in itertools.product(range(m), repeat=n):
        if max(a.count(b) for b in range(m)) > 2:
            continue
        mk = max(sum(l for l, x in zip(loads, a) if x == b) for b in range(m))
        best = mk if best is None else min(best, mk)
    return best


def test_graham_bound_and_brute_force():
    rng = np.random.default_rng(30)
    for trial in range(120):
        m = int(rng.integers(2, 5))
        n = int(rng.integers(1, 11 if m <= 3 else 9))
        loads = rng.integers(0, 60, size=n).tolist()
        _, off, items, load = O.lpt_schedule(loads, m)
        opt = O.brute_force_makespan(loads, m)
        lpt = int(load.max())
        assert opt <= lpt
        assert 3 * m * lpt <= (4 * m - 1) * opt  # LPT <= (4/3 - 1/(3m)) OPT
        assert sorted(items.tolist()) == list(range(n))
        assert load.sum() == sum(loads)
        if n <= 2 * m and n <= 7:
            # classical: greedy is optimal when an optimal schedule with at most
            # two items per machine exists
            if _opt_at_most_two_per_bin(loads, m) == opt:
                assert lpt == opt


def test_brute_force_small_known():
    assert O.brute_force_makespan([3, 3, 2, 2, 2], 2) == 6  # greedy gives 7
    assert int(O.lpt_schedule([3, 3, 2, 2, 2], 2)[3].max()) == 7
    assert O.brute_force_makespan([5], 3) == 5
    assert O.brute_force_makespan([], 3) == 0


def test_fewer_items_than_bins_and_equal_loads():
    bin_of, off, items, load = O.lpt_schedule([4, 9, 1], 5)
    assert bin_of.tolist() == [1, 0, 2]  # largest first into bins 0, 1, 2
    assert load.tolist() == [9, 4, 1, 0, 0]
    bin_of, off, items, load = O.lpt_schedule([7] * 7, 3)
    assert bin_of.tolist() == [0, 1, 2, 0, 1, 2, 0]
    assert off.tolist() == [0, 3, 5, 7]
    assert items.tolist() == [0, 3, 6, 1, 4, 2, 5]


def test_zero_loads_and_errors():
    bin_of, off, items, load = O.lpt_schedule([0, 0, 5], 2)
    assert bin_of.tolist() == [1, 1, 0]  # 5 -> bin0; both zeros -> bin1 (load stays 0 < 5)
    with pytest.raises(ValueError):
        O.lpt_schedule([1], 0)
    with pytest.raises(ValueError):
        O.lpt_schedule([-1], 2)


def test_balance_versus_contiguous_placement():
    """The naive placement the S-HPLB summary contrasts (consecutive heads per
    device) is never better than greedy on these skewed budgets."""
    rng = np.random.default_rng(31)
    for _ in range(50):
        loads = np.exp(rng.uniform(0, 3, 32)).round().astype(int).tolist()
        m = 8
        naive = max(sum(loads[i * 4:(i + 1) * 4]) for i in range(m))
        lpt = int(O.lpt_schedule(loads, m)[3].max())
        assert lpt <= naive
        assert lpt <= sum(loads) / m + max(loads)
