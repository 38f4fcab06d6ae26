"""The host library's calibration (sa_budget_recovery, sa_budget_shift) against
the calibration oracle, bit for bit, and its argument checks.  Needs the built
library (host code only: no GPU)."""

import numpy as np
import pytest

import oracle as O

SA = pytest.importorskip("head_heterogeneous_block_amd.sparse_attn", reason="library not built", exc_type=ImportError)


def _qk(seed, b=1, H=2, Hk=1, S=300, D=16, scale=1.0):
    r = np.random.default_rng(seed)
    q = (scale * r.standard_normal((b, H, S, D))).astype(np.float32)
    k = (scale * r.standard_normal((b, Hk, S, D))).astype(np.float32)
    return q, k


def _budget(H, min_blocks=2):
    return {"min_blocks": [min_blocks] * H, "ratio_q16": [0] * H, "n_sink": [1] * H, "n_local": [1] * H}


def test_host_recovery_and_shift_match_oracle_bitwise():
    q, k = _qk(6, b=2, H=4, Hk=2, S=512, D=32, scale=1.5)
    W32 = O.block_attention_mass(q, k, 64).astype(np.float32)
    bud = _budget(4)
    step = 4096
    got = SA.sa_budget_recovery(W32, bud, step)
    want = O.recovery_table(W32.astype(np.float64), bud, step)
    assert np.array_equal(got, want)
    for per in (step, 4 * step, 8 * step):
        r_host = SA.sa_budget_shift(got, step, 4 * per)
        assert r_host.tolist() == O.maxmin_shift(want, 4 * per, step)


def test_host_calibration_rejects_bad_arguments():
    rec = np.ones((3, 16))
    with pytest.raises(SA.SaError):
        SA.sa_budget_shift(rec, 4096, 3 * 4096 + 1)  # not a whole number of steps per head
    with pytest.raises(SA.SaError):
        SA.sa_budget_shift(rec, 5000, 3 * 5000)  # step does not divide 2^16
    with pytest.raises(SA.SaError):
        SA.sa_budget_recovery(np.ones((1, 2, 3, 3), np.float32), _budget(2, min_blocks=1), 4096)
