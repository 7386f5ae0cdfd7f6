"""The oracle's decode-time pieces against what pins them: in-place compaction
against numpy fancy indexing on a copy, and rescoring of a resident cache against
scoring a contiguous copy of its valid rows (the definition), with garbage --
including non-finite bit patterns -- in the rows past n_valid."""
import numpy as np
import pytest

from attention_perturbation_scoring_amd import workload as wl
from oracle import oracle as orc


def _cache(rng, Hkv, cap, d):
    return wl.bf16_bits(rng.standard_normal((Hkv, cap, d), dtype=np.float32))


def _ascending(rng, n_valid, budget, prefix=0):
    """A strictly ascending keep list of `budget` entries in [0, n_valid) whose
    first `prefix` entries are 0 .. prefix-1 (rows already in place)."""
    rest = rng.choice(np.arange(prefix, n_valid), budget - prefix, replace=False)
    return np.concatenate([np.arange(prefix), np.sort(rest)]).astype(np.int32)


@pytest.mark.parametrize("Hkv,cap,n_valid,d,budget,prefix", [
    (1, 10, 10, 8, 4, 0), (2, 50, 37, 16, 20, 3), (3, 300, 300, 24, 299, 0),
    (2, 64, 40, 8, 40, 0), (1, 200, 150, 32, 75, 10)])
def test_inplace_matches_fancy_indexing(Hkv, cap, n_valid, d, budget, prefix):
    rng = np.random.default_rng(cap + budget)
    cache = _cache(rng, Hkv, cap, d)
    keep = np.stack([_ascending(rng, n_valid, budget, prefix) for _ in range(Hkv)])
    before = cache.copy()
    orc.compact_inplace(cache, keep, n_valid)
    for g in range(Hkv):
        np.testing.assert_array_equal(cache[g, :budget], before[g][keep[g]])
    np.testing.assert_array_equal(cache[:, n_valid:], before[:, n_valid:])


def test_inplace_chains_of_moves():
    """Rows that are both a destination and a later row's source: keep = [1, 3, 4, 6]
    moves 1->0, 3->1, 4->2, 6->3 -- row 1 must be read before it is overwritten."""
    rng = np.random.default_rng(5)
    cache = _cache(rng, 1, 8, 8)
    before = cache.copy()
    keep = np.array([[1, 3, 4, 6]], dtype=np.int32)
    orc.compact_inplace(cache, keep, 8)
    np.testing.assert_array_equal(cache[0, :4], before[0, [1, 3, 4, 6]])


@pytest.mark.parametrize("bad", [[0, 2, 2], [3, 1, 5], [0, 4, 9], [-1, 2, 3]])
def test_inplace_rejects_invalid_lists_and_moves_nothing(bad):
    rng = np.random.default_rng(9)
    cache = _cache(rng, 2, 12, 8)
    before = cache.copy()
    keep = np.array([[0, 1, 2], bad], dtype=np.int32)
    with pytest.raises(orc.OracleError) as e:
        orc.compact_inplace(cache, keep, 9)
    assert e.value.code == orc.ERANGE
    np.testing.assert_array_equal(cache, before)


@pytest.mark.parametrize("Hq,Hkv,d,cap,n_valid,w,pool", [
    (4, 2, 16, 40, 23, 3, 3), (8, 2, 32, 300, 257, 8, 7), (2, 1, 8, 9, 9, 2, 1)])
def test_rescore_is_score_of_the_resident_rows(Hq, Hkv, d, cap, n_valid, w, pool):
    rng = np.random.default_rng(n_valid)
    q = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    k, v = _cache(rng, Hkv, cap, d), _cache(rng, Hkv, cap, d)
    k[:, n_valid:] = 0x7FC1   # NaN bit patterns past the valid rows: never read
    v[:, n_valid:] = 0xFF80   # -inf
    got = orc.rescore(q, k, v, n_valid, pool)
    want = orc.score(q, np.ascontiguousarray(k[:, :n_valid]), np.ascontiguousarray(v[:, :n_valid]), pool)
    np.testing.assert_array_equal(got, want)
    assert np.all(np.isinf(got[:, n_valid - w:]))


def test_decode_cycle():
    """Prefill, evict to the budget in place, append m decode rows, rescore: the
    rescoring equals scoring the compacted-plus-appended rows directly, the window
    (the last w rows) survives, and the cache ends as the kept rows in order."""
    rng = np.random.default_rng(21)
    Hq, Hkv, d, w, pool = 8, 2, 32, 4, 5
    n0, budget, m = 200, 40, 24
    cap = budget + m + 8
    q0 = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    k0, v0 = _cache(rng, Hkv, n0, d), _cache(rng, Hkv, n0, d)
    keep0 = orc.select(orc.score(q0, k0, v0, pool), budget)
    k, v = np.zeros((Hkv, cap, d), np.uint16), np.zeros((Hkv, cap, d), np.uint16)
    k[:, :budget], v[:, :budget] = orc.compact(k0, keep0), orc.compact(v0, keep0)
    k[:, budget:budget + m], v[:, budget:budget + m] = _cache(rng, Hkv, m, d), _cache(rng, Hkv, m, d)
    n_valid = budget + m
    q1 = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    s1 = orc.rescore(q1, k, v, n_valid, pool)
    np.testing.assert_array_equal(
        s1, orc.score(q1, np.ascontiguousarray(k[:, :n_valid]), np.ascontiguousarray(v[:, :n_valid]), pool))
    keep1 = orc.select(s1, budget)
    for g in range(Hkv):
        assert set(range(n_valid - w, n_valid)) <= set(keep1[g].tolist())
    kb, vb = k.copy(), v.copy()
    orc.compact_inplace(k, keep1, n_valid)
    orc.compact_inplace(v, keep1, n_valid)
    for g in range(Hkv):
        np.testing.assert_array_equal(k[g, :budget], kb[g][keep1[g]])
        np.testing.assert_array_equal(v[g, :budget], vb[g][keep1[g]])
