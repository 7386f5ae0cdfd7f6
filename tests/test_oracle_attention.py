"""Pins of the oracle's attention-only (SnapKV-style) scores.

The pages give the score as MaxPool1d over the window-summed attention weights
("paper tables", Table 14, SnapKV row) with DropKV's observation window and
pooling kernel ("paper digest", App. B).  These checks tie the oracle to facts
other than its own code: probabilities of each query sum to one, a zero query
attends uniformly (closed form with the tail-causal limit), and a pure-Python
brute force on tiny inputs.
"""
import numpy as np
import pytest

from attention_perturbation_scoring_amd import workload as wl
from oracle import oracle as orc
import brute


def _rand(rng, Hq, Hkv, w, d, n, scale=1.0):
    q = wl.bf16_bits(rng.standard_normal((Hq, w, d)).astype(np.float32) * scale)
    k = wl.bf16_bits(rng.standard_normal((Hkv, n, d)).astype(np.float32))
    return q, k


@pytest.mark.parametrize("Hq,Hkv,w,d,n", [(1, 1, 1, 8, 5), (4, 2, 3, 8, 22), (8, 2, 4, 16, 40),
                                          (6, 3, 2, 8, 9)])
def test_rows_sum_to_window_length(Hq, Hkv, w, d, n):
    """Each query's probabilities sum to 1, so a head's raw scores sum to w."""
    rng = np.random.default_rng(Hq * 100 + n)
    q, k = _rand(rng, Hq, Hkv, w, d, n, scale=2.0)
    raw = orc.attention_raw(q, k)
    np.testing.assert_allclose(raw.sum(axis=1), np.full(Hkv, float(w)), rtol=1e-13)
    assert np.all(raw >= 0)


@pytest.mark.parametrize("w,n", [(1, 7), (3, 10), (5, 5)])
def test_zero_query_is_uniform_with_causal_limit(w, n):
    """q = 0: query t attends uniformly to its n-w+t+1 visible keys."""
    Hq = Hkv = 2
    d = 8
    q = np.zeros((Hq, w, d), np.uint16)
    rng = np.random.default_rng(5)
    _, k = _rand(rng, Hq, Hkv, w, d, n)
    raw = orc.attention_raw(q, k)
    want = np.zeros(n)
    for t in range(w):
        P = n - w + t
        want[: P + 1] += 1.0 / (P + 1)
    for g in range(Hkv):
        np.testing.assert_allclose(raw[g], want, rtol=1e-14)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    q, k = _rand(rng, 4, 2, 3, 8, 13, scale=3.0)
    np.testing.assert_allclose(orc.attention_raw(q, k), brute.attention_raw(q, k), rtol=1e-12,
                               atol=1e-300)


def test_scores_pool_and_protect():
    """The final scores are the shared MaxPool + protection of the raw sums."""
    rng = np.random.default_rng(9)
    q, k = _rand(rng, 4, 2, 3, 8, 30, scale=2.0)
    raw = orc.attention_raw(q, k)
    s = orc.attention_score(q, k, 5)
    np.testing.assert_array_equal(s, orc.pool_protect(raw, 3, 5))
    assert np.all(np.isinf(s[:, -3:]))


def test_nonfinite_rejected():
    rng = np.random.default_rng(1)
    q, k = _rand(rng, 2, 1, 2, 8, 6)
    k[0, 2, 3] = 0x7F80   # +inf
    with pytest.raises(orc.OracleError) as e:
        orc.attention_raw(q, k)
    assert e.value.code == 3


def test_window_lse_against_logsumexp_and_closed_form():
    """Window LSE: torch's float64 logsumexp over the tail-causal logits, and
    log(n-w+t+1) exactly for a zero query."""
    import torch
    rng = np.random.default_rng(4)
    Hq, Hkv, w, d, n = 4, 2, 3, 16, 25
    q, k = _rand(rng, Hq, Hkv, w, d, n, scale=2.0)
    got = orc.window_lse(q, k)
    qf = torch.from_numpy(wl.bf16_to_f32(q).astype(np.float64))
    kf = torch.from_numpy(wl.bf16_to_f32(k).astype(np.float64))
    G = Hq // Hkv
    for h in range(Hq):
        for t in range(w):
            P = n - w + t
            logits = kf[h // G, : P + 1] @ qf[h, t] / np.sqrt(d)
            assert abs(got[h, t] - float(torch.logsumexp(logits, 0))) <= 1e-12 * max(1.0, abs(got[h, t]))
    z = orc.window_lse(np.zeros_like(q), k)
    for t in range(w):
        np.testing.assert_allclose(z[:, t], np.log(n - w + t + 1), rtol=1e-15)
