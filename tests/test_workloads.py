"""The synthetic budget generator's three readings of the fixed-total shift
(an input convention, not the method): every fit keeps the target mean (up to
the 2^-16 quantisation) and the draw order of the heads; "clamp" keeps every
ratio inside the stated range, "span" reaches both ends of it."""

import numpy as np
import pytest

from head_heterogeneous_block_amd import workloads as W


@pytest.mark.parametrize("spec", [W.LLAMA_32K, W.LLAMA_128K], ids=lambda s: s.name)
@pytest.mark.parametrize("fit", ["rescale", "clamp", "span"])
def test_budget_fits(spec, fit):
    sp = spec.with_(budget_fit=fit)
    r = np.asarray(W.prefill_budgets(sp, W.seed_of(spec))["ratio_q16"], dtype=np.float64) / 65536.0
    base = np.asarray(W.prefill_budgets(spec, W.seed_of(spec))["ratio_q16"], dtype=np.float64)
    assert abs(r.mean() - spec.mean) <= 1.0 / 65536.0
    # the same heads are heavy and light: the fit is monotone in the draw
    order = np.argsort(base, kind="stable")
    assert np.all(np.diff(r[order]) >= -1.0 / 65536.0)
    if fit == "clamp":
        q = 0.5 / 65536.0  # the quantisation of the ratios
        assert r.min() >= spec.lo - q and r.max() <= spec.hi + q
    if fit == "span":
        assert abs(r.min() - spec.lo) <= 0.5 / 65536.0 and abs(r.max() - spec.hi) <= 0.5 / 65536.0


def test_budget_fit_rejects_unknown():
    with pytest.raises(ValueError):
        W.prefill_budgets(W.LLAMA_32K.with_(budget_fit="other"), 1)
    with pytest.raises(ValueError):
        W.prefill_budgets(W.LLAMA_32K.with_(budget_fit="clamp", mean=0.9), 1)
