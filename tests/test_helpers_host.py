"""Host checks of the parity-test helpers (no GPU)."""

import numpy as np
import pytest

from fenwick_tree_hierarchical_amd.workloads import WORKLOADS, make_inputs
from oracle import forms
from tests.helpers import ROW_FACTOR, OraclePool, parity


def test_oracle_pool_equals_the_recurrence():
    x = make_inputs(WORKLOADS["small_bf16"], B=2, H=3, T=70, d=16, variant="weak_decay", seed=9)
    ref, _ = forms.forward_recurrent(x["q"], x["k"], x["v"], x["lam"], log_a=x["log_a"])
    got = OraclePool(x, workers=2).result(120)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_parity_sees_one_wrong_row_and_one_wrong_head():
    rng = np.random.default_rng(0)
    ref = rng.normal(size=(2, 3, 2698, 64))
    got = ref * (1 + 1e-3 * rng.normal(size=ref.shape))
    p = parity(got, ref)
    assert p["whole"] < 2e-3 and p["head"] < 2e-3 and p["row"] < 1e-2
    bad = got.copy()
    bad[1, 2, 1234] = -ref[1, 2, 1234]          # one row entirely wrong
    p = parity(bad, ref)
    assert p["whole"] < 2e-2                    # hidden under the whole-tensor norm
    assert p["row"] > ROW_FACTOR * 2e-2 and tuple(p["worst_row"])[1] == 1234
    bad = got.copy()
    bad[0, 1] *= 1.1                            # one head 10 % off
    p = parity(bad, ref)
    assert p["whole"] < 5e-2 and p["head"] > 9e-2 and tuple(p["worst_head"]) == (0, 1)


def test_a_single_row_head_is_held_to_the_row_bar():
    from tests.helpers import ROW_FACTOR, assert_parity
    ref = np.ones((8, 1, 8))
    got = ref.copy()
    got[0, 0] *= 1.03                     # 3 % off: above the head bar, below the row bar
    assert_parity(got, ref, 0.02, "one row", lead=1)
    ref2 = np.ones((8, 2, 8))
    got2 = ref2.copy()
    got2[0] *= 1.03                       # a two-row head 3 % off fails the head bar
    with pytest.raises(AssertionError):
        assert_parity(got2, ref2, 0.02, "two rows", lead=1)
    assert ROW_FACTOR * 0.02 > 0.03
