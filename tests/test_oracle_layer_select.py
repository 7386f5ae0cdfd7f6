"""Pins of the oracle's layer-wide (cross-head budget) selection: a full numpy
sort on (score, head, index), disjoint per-head score ranges (closed-form
counts), and the window guarantee from +inf protection."""
import numpy as np
import pytest

from oracle import oracle as orc


def _sort_select(s, budget):
    Hkv, n = s.shape
    g = np.repeat(np.arange(Hkv), n)
    j = np.tile(np.arange(n), Hkv)
    flat = s.reshape(-1)
    order = np.lexsort((j, g, flat))          # ascending (score, head, index)
    kept = np.sort(order[Hkv * n - budget:])
    return kept.astype(np.int32), np.bincount(kept // n, minlength=Hkv).astype(np.int32)


@pytest.mark.parametrize("Hkv,n,budget", [(1, 10, 4), (3, 17, 20), (4, 50, 1), (5, 8, 40), (2, 30, 0)])
def test_matches_full_sort_with_ties(Hkv, n, budget):
    rng = np.random.default_rng(Hkv * 1000 + n)
    s = rng.integers(0, 5, size=(Hkv, n)).astype(np.float64)
    s[:, : n // 3] = rng.random((Hkv, n // 3))
    keep, counts = orc.select_layer(s, budget)
    want_keep, want_counts = _sort_select(s, budget)
    np.testing.assert_array_equal(keep, want_keep)
    np.testing.assert_array_equal(counts, want_counts)
    assert counts.sum() == budget


def test_disjoint_head_ranges_fill_the_top_heads_first():
    """Head g's scores lie in [g, g+1): the survivors are the top heads whole,
    then the largest scores of the next head down."""
    Hkv, n = 4, 25
    rng = np.random.default_rng(2)
    s = np.arange(Hkv)[:, None] + rng.random((Hkv, n)) * 0.99
    budget = 2 * n + 7
    keep, counts = orc.select_layer(s, budget)
    np.testing.assert_array_equal(counts, [0, 7, n, n])
    top1 = np.argsort(s[1])[-7:]
    np.testing.assert_array_equal(np.sort(keep[:7] - n), np.sort(top1))


def test_protected_windows_survive():
    Hkv, n, w = 3, 40, 4
    rng = np.random.default_rng(7)
    s = rng.random((Hkv, n))
    s[:, -w:] = np.inf
    keep, counts = orc.select_layer(s, Hkv * w + 5)
    assert np.all(counts >= w)
    for g in range(Hkv):
        assert set(range(g * n + n - w, (g + 1) * n)) <= set(keep.tolist())
