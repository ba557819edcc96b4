"""Pins for the oracle's Fenwick level function (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import levels

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bucket_counts.json")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 16, 17, 64, 100, 256, 1024])
def test_walk_equals_closed_form(T):
    assert np.array_equal(levels.level_table_walk(T), levels.level_table(T))


def test_scalar_level_matches_table():
    tab = levels.level_table(200)
    for t in range(200):
        for s in range(t + 1):
            assert levels.level(t, s) == tab[t, s]


def test_bucket_invariants_up_to_8192():
    """Partition of [0,t], sizes 1 and 2^(l-1), count bound, age monotonicity."""
    for t in range(8192):
        bk = levels.walk_buckets(t)
        covered = np.zeros(t + 1, dtype=np.int64)
        for lev, lo, hi in bk:
            covered[lo:hi] += 1
            assert hi - lo == (1 if lev == 0 else 2 ** (lev - 1))
        assert np.all(covered == 1)                                  # partition
        assert len(bk) == 1 + bin(t).count("1")
        assert len(bk) <= math.ceil(math.log2(t + 1)) + 1            # O(log t) states
        levs = [lev for lev, _, _ in bk]
        assert levs == sorted(levs)                                 # newest first
        assert [lev for lev in levs] == levels.active_levels(t)


def test_levels_never_decrease_with_age():
    tab = levels.level_table(512).astype(np.int64)
    for t in range(512):
        row = tab[t, : t + 1][::-1]                                  # newest -> oldest
        assert np.all(np.diff(row) >= 0)


@pytest.mark.parametrize("C", [2, 4, 8, 16, 32, 64, 128])
def test_chunk_factorisation(C):
    """Inside a chunk the level depends on the in-chunk offsets only; across
    chunks it is log2(C) + 1 + msb(chunk_t xor chunk_s)."""
    T = 4 * C + C // 2
    tab = levels.level_table(T).astype(np.int64)
    lc = int(math.log2(C))
    for t in range(T):
        for s in range(t + 1):
            ct, cs = t // C, s // C
            if ct == cs:
                exp = levels.level(t % C, s % C)
            else:
                exp = lc + 1 + (ct ^ cs).bit_length() - 1
            assert tab[t, s] == exp


def test_num_levels_matches_workload_table():
    for T, L in [(64, 7), (2048, 12), (16384, 15), (131072, 18), (33024, 17), (1, 1), (2, 2), (3, 3)]:
        assert levels.num_levels(T) == L
        assert levels.level_table(min(T, 2048), rows=[min(T, 2048) - 1]).max() <= L - 1


def test_golden_bucket_counts_from_pages():
    g = json.load(open(GOLDEN))
    for case in g["max_buckets"]:
        n = case["tokens"]
        # max over t < n of the bucket count: the walk itself for small n; for
        # large n the count 1 + popcount(t) (equal to the walk's count, see the
        # invariant test) evaluated for every t < n.
        if n <= 5000:
            best = max(len(levels.walk_buckets(t)) for t in range(n))
        else:
            best = int(np.bitwise_count(np.arange(n, dtype=np.uint64)).max()) + 1
        assert best == case["about_buckets"], case
    sizes = [hi - lo for lev, lo, hi in levels.walk_buckets(63) if lev >= 1]
    assert sizes == g["bucket_sizes_newest_first"]["sizes"]
