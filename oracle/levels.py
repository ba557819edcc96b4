"""Fenwick-tree bucket levels (oracle; test infrastructure only).

[LLA-it] Sommario tecnico section 2, item 1 (hierarchical partition with a
Fenwick / binary indexed tree): the prefix seen by a query is cut into buckets
whose sizes grow by powers of two, recent tokens in small buckets and old
tokens in large ones.  [LLA-es] Resumen tecnico section 2, "Conceptos clave",
says the same and adds that O(log T) states are touched per step.  The lay
parts of both pages describe the same boxes: the newest tokens one by one,
then groups of 2, 4, 8, ... ([LLA-es] "Lo esencial", item 2), and about 10
boxes for 1,000 tokens and about 20 for 1,000,000 ([LLA-it] "L'essenziale",
box metaphor; [LLA-es] "Lo esencial", item 3).

Reading (the pages print no formula): query t itself is bucket 0; the strict
prefix [0, t) is split by repeatedly stripping the lowest set bit of t -- the
set bit k of t yields a bucket of the 2^k keys just older than the previous
bucket, at level k + 1.  Two derivations follow and are tested against each
other and against the invariants the pages state:

  * ``walk_buckets``   -- the lowest-set-bit walk, literally;
  * ``level``          -- closed form l(t, s) = 1 + msb(t xor s) for s < t.

Pins: walk == closed form for every pair up to T = 1024; bucket sizes 1 and
2^(l-1); the buckets partition [0, t]; at most 1 + popcount(t) <=
ceil(log2(t+1)) + 1 buckets; levels never decrease with the age of the key;
the maximum bucket count over prefixes of 1,000 and 1,000,000 tokens equals the
pages' "about 10" and "about 20" (tests/golden/bucket_counts.json).
"""

from __future__ import annotations

import numpy as np


def level(t: int, s: int) -> int:
    """Bucket level of key ``s`` seen from query ``t`` (closed form).

    0 for s == t; 1 + index of the highest bit where t and s differ for
    s < t.  Undefined (raises) for s > t: the future is not in any bucket.
    """
    if s > t or s < 0:
        raise ValueError("key must satisfy 0 <= s <= t")
    if s == t:
        return 0
    return (t ^ s).bit_length()


def walk_buckets(t: int) -> list[tuple[int, int, int]]:
    """Buckets of query ``t`` as (level, first_key, end_key_exclusive).

    Built by the Fenwick walk: start at ``b = t``; while ``b > 0`` take its
    lowest set bit 2^k, emit keys [b - 2^k, b) at level k + 1 and clear that
    bit.  Key t itself is emitted first as the level-0 bucket.  Ordered from
    the newest bucket to the oldest.
    """
    out = [(0, t, t + 1)]
    b = t
    while b > 0:
        low = b & (-b)
        k = low.bit_length() - 1
        out.append((k + 1, b - low, b))
        b -= low
    return out


def level_table_walk(T: int) -> np.ndarray:
    """int8 [T, T] level table from the walk; -1 where s > t."""
    tab = np.full((T, T), -1, dtype=np.int8)
    for t in range(T):
        for lev, lo, hi in walk_buckets(t):
            tab[t, lo:hi] = lev
    return tab


def level_table(T: int, rows: np.ndarray | None = None) -> np.ndarray:
    """int8 level table from the closed form; -1 where s > t.

    ``rows`` selects query indices (default: all ``T``); the result is
    [len(rows), T].
    """
    t = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    s = np.arange(T, dtype=np.int64)
    x = t[:, None] ^ s[None, :]
    # bit_length of a non-negative int64, vectorised: count shifts until zero.
    bl = np.zeros_like(x)
    y = x.copy()
    while np.any(y):
        nz = y != 0
        bl[nz] += 1
        y >>= 1
    tab = bl.astype(np.int8)
    tab[s[None, :] > t[:, None]] = -1
    return tab


def num_levels(T: int) -> int:
    """Levels needed for sequences of length T: ceil(log2 T) + 1 (T >= 1).

    The largest level any pair reaches is 1 + msb(T - 1) = bit_length(T-1).
    """
    if T < 1:
        raise ValueError("T >= 1")
    return (T - 1).bit_length() + 1


def active_levels(t: int) -> list[int]:
    """Levels holding at least one key for query ``t``: 0 and every l >= 1
    whose bit l-1 is set in t (from the walk: set bit k -> level k+1)."""
    return [0] + [k + 1 for k in range(t.bit_length()) if (t >> k) & 1]
