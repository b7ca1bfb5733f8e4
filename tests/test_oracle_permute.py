"""Pins of the oracle's dispatch permutation (expert_mask -> one token
dispatch flow; on one device the expert-parallel all-to-all is a permutation
of token copies grouped by expert).

Invariants: counts equal the histogram (np.bincount); offsets are its
exclusive prefix sum; dest is a bijection onto the filled rows; every row of
expert e's segment holds a token routed to e, tokens ascending (stable);
library special case np.argsort(kind="stable"); gathered rows are byte copies.
"""
import numpy as np
import pytest


def _random_ids(rng, T, E, k):
    return np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (64, 8, 2), (300, 16, 4), (1000, 384, 6),
                                   (257, 5, 5)])
def test_permutation_invariants(orc, T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    ids = _random_ids(rng, T, E, k)
    counts, offsets, dest, src, flags = orc.permute(ids, E)
    assert flags == 0
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(offsets[1:], np.cumsum(counts))
    N = T * k
    assert np.array_equal(np.sort(dest), np.arange(N))          # bijection
    assert np.array_equal(src[dest], np.arange(N) // k)          # row holds its token
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                          # stable, distinct
        assert np.all((ids[seg] == e).any(axis=1))
    order = np.argsort(flat, kind="stable")                      # library special case
    inv = np.empty(N, np.int64)
    inv[dest] = np.arange(N)
    assert np.array_equal(inv, order)


def test_duplicate_ids_in_a_row(orc):
    # a table row may repeat an expert: each copy gets its own row, in slot order
    ids = np.array([[3, 3], [1, 3]], np.int32)
    counts, offsets, dest, src, _ = orc.permute(ids, 4)
    assert counts.tolist() == [0, 1, 0, 3]
    assert dest.tolist() == [1, 2, 0, 3]
    assert src.tolist() == [1, 0, 0, 1]


def test_invalid_ids_dropped(orc):
    ids = np.array([[0, 5], [-1, 1], [1, 0]], np.int32)
    counts, offsets, dest, src, flags = orc.permute(ids, 4)
    assert flags == orc.FLAG_BAD_EXPERT_ID
    assert counts.tolist() == [2, 2, 0, 0]
    assert offsets[-1] == 4
    assert dest.tolist() == [0, -1, -1, 2, 3, 1]
    assert src.tolist() == [0, 2, 1, 2, -1, -1]


def test_gather_copies_rows(orc):
    rng = np.random.default_rng(3)
    T, d, E, k = 50, 64, 8, 3
    x = rng.integers(0, 65536, (T, d)).astype(np.uint16)
    ids = _random_ids(rng, T, E, k)
    _, _, dest, src, _ = orc.permute(ids, E)
    xp = orc.gather(x, src)
    assert np.array_equal(xp, x[src])
    assert np.array_equal(xp[dest], np.repeat(x, k, axis=0))
