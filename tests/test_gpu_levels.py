"""Level tables from the device are byte-identical to the oracle's (GPU)."""

import numpy as np
import pytest

from oracle import levels
from tests.helpers import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,C", [(1, 16), (17, 4), (64, 16), (100, 16), (1000, 1), (2048, 64), (4096, 128),
                                 (4096, 2)])
def test_level_table_full(T, C):
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    say(f"level table T={T} C={C}")
    tab = la.loglinear_level_table(T, C, dev).cpu().numpy()
    assert np.array_equal(tab, levels.level_table(T))


@pytest.mark.parametrize("C", [16, 64, 128])
def test_level_table_sampled_rows_16k(C):
    dev = need_gpu()
    import fenwick_tree_hierarchical_amd as la
    T = 16384
    say(f"level table T={T} C={C} (sampled rows)")
    tab = la.loglinear_level_table(T, C, dev)
    rng = np.random.default_rng(C)
    rows = np.unique(np.concatenate([[0, 1, C - 1, C, T - 1, T // 2, T // 2 - 1], rng.integers(0, T, 48)]))
    got = tab[rows].cpu().numpy()
    assert np.array_equal(got, levels.level_table(T, rows=rows))
