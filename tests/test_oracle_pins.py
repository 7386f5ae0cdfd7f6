"""Pins of the float64 oracle against things other than itself (CPU only).

Each test cites the passage it checks (DropKV, arXiv 2610.22130, as described
on the studied pages) and is chosen so that a plausible slip in the oracle -- a
dropped term, a wrong sign or index, a swapped operand, a wrong causal limit,
a wrong head mapping -- fails at least one of them.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

from attention_perturbation_scoring_amd import workload as wl
from oracle import oracle as orc
import brute


def _tiny_inputs(seed, Hq, Hkv, d, n, w, scale=1.0):
    rng = np.random.default_rng(seed)
    q = wl.bf16_bits(scale * rng.standard_normal((Hq, w, d), dtype=np.float32))
    k = wl.bf16_bits(scale * rng.standard_normal((Hkv, n, d), dtype=np.float32))
    v = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    return q, k, v


# --- Section 3.1 / Appendix C.2: Delta_j is the change of the output when token j
# --- is deleted and the softmax renormalised.  Brute force by actual deletion.
@pytest.mark.parametrize("Hq,Hkv,w", [(1, 1, 1), (2, 1, 3), (4, 2, 3), (4, 1, 2), (8, 2, 4)])
def test_raw_scores_equal_actual_deletion(Hq, Hkv, w):
    q, k, v = _tiny_inputs(100 + Hq * 10 + w, Hq, Hkv, d=8, n=19, w=w)
    got = orc.raw_scores(q, k, v)
    want = brute.deletion_raw(q, k, v)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=0)


def test_raw_scores_equal_actual_deletion_tiny_config():
    cfg = wl.TINY
    inp = wl.make_layer(cfg, cfg.seed, accept=lambda q, k, v: orc.max_probability(q, k, v) <= 0.5)
    got = orc.raw_scores(inp["q"], inp["k"], inp["v"])
    want = brute.deletion_raw(inp["q"], inp["k"], inp["v"])
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=0)


# --- softmax and output against library routines (torch, float64, explicit tail mask)
def test_window_attention_matches_torch():
    q, k, v = _tiny_inputs(5, 4, 2, d=16, n=30, w=4)
    p, a, sx = orc.window_attention(q, k, v)
    qf, Kh, Vh, G = brute.expand_heads(q, k, v)
    Hq, w, d = qf.shape
    n = Kh.shape[1]
    Q = torch.from_numpy(qf)
    Kt, Vt = torch.from_numpy(Kh), torch.from_numpy(Vh)
    logits = Q @ Kt.transpose(1, 2) / math.sqrt(d)          # [Hq][w][n]
    pos = torch.arange(n)[None, :]
    qpos = (n - w + torch.arange(w))[:, None]
    logits = logits.masked_fill(pos > qpos, float("-inf"))
    pt = torch.softmax(logits, dim=-1)
    np.testing.assert_allclose(p, pt.numpy(), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(a, (pt @ Vt).numpy(), rtol=1e-11, atol=1e-14)
    # the last window query sees every key: plain attention with no mask
    full = torch.nn.functional.scaled_dot_product_attention(
        Q[:, -1:, :], Kt, Vt, scale=1.0 / math.sqrt(d))
    np.testing.assert_allclose(a[:, -1, :], full[:, 0, :].numpy(), rtol=1e-10, atol=1e-13)
    # S_excl = sum of non-maximal e_j in units of the maximum
    pm = p.max(axis=-1)
    np.testing.assert_allclose(sx, (1.0 - pm) / pm, rtol=1e-10)


# --- closed form: q = 0 gives uniform attention over the N_t = n-w+t+1 visible keys,
# --- so Delta_j = (a_t - v_j)/(N_t - 1) exactly (Section 3.1); exact rationals.
@pytest.mark.parametrize("Hq,Hkv,n,w", [(1, 1, 6, 1), (2, 1, 7, 3), (4, 2, 9, 2)])
def test_uniform_attention_closed_form(Hq, Hkv, n, w):
    d = 3
    rng = np.random.default_rng(n * 31 + w)
    vint = rng.integers(-8, 9, size=(Hkv, n, d))
    v = wl.bf16_bits(vint.astype(np.float32))
    q = np.zeros((Hq, w, d), dtype=np.uint16)
    k = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    got = orc.raw_scores(q, k, v)
    for g in range(Hkv):
        for j in range(n):
            want = Fraction(0)
            for t in range(w):
                N = n - w + t + 1
                if j >= N:
                    continue
                a = [Fraction(int(sum(vint[g, i, c] for i in range(N))), N) for c in range(d)]
                dist2 = sum((a[c] - int(vint[g, j, c])) ** 2 for c in range(d))
                want += dist2 / Fraction((N - 1) ** 2)
            # all G heads of the group are identical, so the mean is the single-head value
            assert got[g, j] == pytest.approx(float(want), rel=1e-13, abs=1e-300), (g, j)


# --- Section 3.3: with w = 1 the score is ||Delta_j||^2, so the ranking equals the
# --- ranking by ||Delta_j|| from actual deletion; G identical heads average to one.
def test_w1_ranking_and_identical_heads():
    q1, k, v = _tiny_inputs(77, 1, 1, d=8, n=25, w=1)
    raw = orc.raw_scores(q1, k, v)[0]
    qf, Kh, Vh, _ = brute.expand_heads(q1, k, v)
    keys = np.arange(25)
    _, a = brute.attend(qf[0, 0], Kh[0], Vh[0], keys)
    norms = np.array([np.linalg.norm(brute.attend(qf[0, 0], Kh[0], Vh[0], keys[keys != j])[1] - a)
                      for j in keys])
    assert list(np.argsort(raw, kind="stable")) == list(np.argsort(norms, kind="stable"))
    q4 = np.repeat(q1, 4, axis=0)   # four identical query heads on one KV head
    np.testing.assert_allclose(orc.raw_scores(q4, k, v)[0], raw, rtol=1e-14)


# --- Section 3.2 with k = 1: the proxy is exact, F({j})^2 = G * raw_j.
def test_k1_proxy_is_exact():
    q, k, v = _tiny_inputs(9, 4, 2, d=8, n=16, w=3)
    raw = orc.raw_scores(q, k, v)
    G = 2
    for g in range(2):
        F2 = np.array([brute.joint_objective_sq(q, k, v, g, [j]) for j in range(16)])
        np.testing.assert_allclose(F2, G * raw[g], rtol=1e-9)
        assert int(np.argmin(F2)) == int(np.argmin(raw[g]))


# --- Section 4 (Theorem 1) and Appendix C.2 (Proposition 1): under the cone
# --- condition and small weights, F(J_hat) <= sqrt(G w) F(J*) / [c (1-eps)(1-k eps)].
def _cone_case(seed, Hq, Hkv, w, n, d=8):
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    q32 = rng.standard_normal((Hq, w, d), dtype=np.float32)
    k32 = (0.5 * rng.standard_normal((Hkv, n, d))).astype(np.float32)
    v32 = (0.3 * rng.standard_normal((Hkv, n, d))).astype(np.float32)
    for g in range(Hkv):
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        Qg = q32[g * G:(g + 1) * G].reshape(-1, d).astype(np.float64)
        b, *_ = np.linalg.lstsq(Qg, np.full(G * w, 3.0 * np.sqrt(d)), rcond=None)
        k32[g, 0] += b.astype(np.float32)          # anchor token 0: logit +3 for every query
        v32[g, 0] = (4.0 * u).astype(np.float32)
    return wl.bf16_bits(q32), wl.bf16_bits(k32), wl.bf16_bits(v32)


@pytest.mark.parametrize("seed,Hq,Hkv,w,n,kk", [(3, 1, 1, 1, 21, 7), (4, 1, 1, 1, 21, 7),
                                                (5, 2, 1, 2, 22, 6)])
def test_theorem1_bound_by_brute_force(seed, Hq, Hkv, w, n, kk):
    q, k, v = _cone_case(seed, Hq, Hkv, w, n)
    raw = orc.raw_scores(q, k, v)[0]
    p, a, _ = orc.window_attention(q, k, v)
    G = Hq // Hkv
    cand = np.arange(1, n - w)                     # history minus the anchor
    # certified constants over every (h, t): c from u = mean unit residual, eps = max p
    vf = brute.widen(v)[0]
    c_all, eps = [], 0.0
    for h in range(Hq):
        for t in range(w):
            r = a[h, t][None, :] - vf[cand]
            unit = r / np.linalg.norm(r, axis=1, keepdims=True)
            u = unit.mean(axis=0)
            u /= np.linalg.norm(u)
            c_all.append(float((unit @ u).min()))
            eps = max(eps, float(p[h, t, cand].max()))
    c = min(c_all)
    assert c > 0 and 1 - kk * eps > 0, (c, eps)
    J_hat = cand[np.argsort(raw[cand], kind="stable")[:kk]]
    subsets, F2 = brute.all_subsets_objective_sq(q, k, v, 0, cand, kk)
    F_opt = math.sqrt(F2.min())
    F_hat = math.sqrt(brute.joint_objective_sq(q, k, v, 0, J_hat))
    ratio = F_hat / F_opt
    bound = math.sqrt(G * w) / (c * (1 - eps) * (1 - kk * eps))
    assert 1.0 - 1e-12 <= ratio <= bound, (ratio, bound)


# --- MaxPool1D as in the third-party notes' Algorithm 1, against torch.
@pytest.mark.parametrize("pool", [1, 3, 5, 7])
def test_pool_matches_torch_and_window_is_inf(pool):
    rng = np.random.default_rng(pool)
    raw = rng.random((3, 40)) * (rng.random((3, 40)) > 0.3)
    w = 5
    got = orc.pool_protect(raw, w, pool)
    r = (pool - 1) // 2
    want = torch.nn.functional.max_pool1d(torch.from_numpy(raw)[:, None, :], pool, 1, r)[:, 0]
    np.testing.assert_array_equal(got[:, :-w], want.numpy()[:, :-w])
    assert np.all(np.isinf(got[:, -w:])) and np.all(got[:, -w:] > 0)


# --- selection: evict the k smallest by (score, index), keep ascending.
@pytest.mark.parametrize("budget", [5, 9, 17, 40])
def test_select_matches_full_sort_with_ties(budget):
    rng = np.random.default_rng(budget)
    s = rng.integers(0, 6, size=(4, 40)).astype(np.float64)   # many ties
    s[:, -5:] = np.inf
    got = orc.select(s, budget)
    np.testing.assert_array_equal(got, brute.sort_select(s, budget))
    # the protected window survives whenever budget >= w
    for g in range(4):
        assert set(range(35, 40)) <= set(got[g].tolist())


def test_select_budget_n_and_budget_w():
    s = np.random.default_rng(1).random((2, 30))
    s[:, -4:] = np.inf
    np.testing.assert_array_equal(orc.select(s, 30), np.tile(np.arange(30, dtype=np.int32), (2, 1)))
    np.testing.assert_array_equal(orc.select(s, 4), np.tile(np.arange(26, 30, dtype=np.int32), (2, 1)))


def test_compact_is_fancy_indexing():
    rng = np.random.default_rng(2)
    x = rng.integers(0, 65535, size=(3, 50, 8), dtype=np.uint16)
    keep = np.sort(np.stack([rng.choice(50, 10, replace=False) for _ in range(3)]), axis=1).astype(np.int32)
    got = orc.compact(x, keep)
    np.testing.assert_array_equal(got, np.stack([x[g][keep[g]] for g in range(3)]))


# --- singular rows are rejected, not epsilon-patched (third-party notes, Algorithm 1)
def _peaked(n, d, L, seed=0):
    """One query, one head: key 0 has logit L, every other key logit 0 (d = 8)."""
    rng = np.random.default_rng(seed)
    q = np.zeros((1, 1, d), dtype=np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((1, n, d), dtype=np.float32)
    k[0, :, 1:] = rng.standard_normal((n, d - 1))
    k[0, 0, 0] = L * math.sqrt(d)
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    return wl.bf16_bits(q), wl.bf16_bits(k), wl.bf16_bits(v)


def test_singular_row_rejected():
    q, k, v = _peaked(12, 8, 60.0)
    with pytest.raises(orc.OracleError) as e:
        orc.raw_scores(q, k, v)
    assert e.value.code == orc.ESINGULAR


@pytest.mark.parametrize("pstar", [0.9, 0.999, 1 - 1e-9])
def test_near_singular_rows_accepted_and_exact(pstar):
    n, d = 12, 8
    L = math.log(pstar * (n - 1) / (1 - pstar))
    q, k, v = _peaked(n, d, L, seed=3)
    got = orc.raw_scores(q, k, v)[0]
    p, _, _ = orc.window_attention(q, k, v)
    # bf16 rounding of the key moves p* slightly; 1 - p* stays within a factor of 3
    assert 1 / 3 < (1 - p.max()) / (1 - pstar) < 3
    want = brute.deletion_raw(q, k, v)[0]
    # the arg-max token's perturbation is O(1): tight agreement
    assert got[0] == pytest.approx(want[0], rel=1e-9)
    # other tokens carry p_j ~ (1 - p*)/(n-1); brute-force subtraction loses digits
    np.testing.assert_allclose(got[1:], want[1:], rtol=max(1e-9, 1e-14 / (1 - pstar)))


def test_nonfinite_inputs_rejected():
    q, k, v = _tiny_inputs(1, 2, 1, d=8, n=10, w=2)
    for arr, val in ((k, 0x7F80), (v, 0x7FC0), (q, 0xFF80)):
        bad = arr.copy()
        bad.reshape(-1)[3] = val
        args = [q, k, v]
        args[[id(q), id(k), id(v)].index(id(arr))] = bad
        with pytest.raises(orc.OracleError) as e:
            orc.raw_scores(*args)
        assert e.value.code == orc.ENONFINITE


def _status(f, *args):
    try:
        f(*args)
        return orc.OK
    except orc.OracleError as e:
        return e.code


def test_input_contract_boundary():
    """Reading R-11: an element of magnitude 2^48 or more (bf16 bits 0x5780 and up,
    either sign) makes the call ERANGE; the largest bf16 below it does not."""
    q, k, v = _tiny_inputs(2, 1, 1, d=8, n=10, w=2)
    for which in ("q", "k", "v"):
        for val in (0x5780, 0xD780, 0x7F7F):
            arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            arrs[which].reshape(-1)[5] = val
            assert _status(orc.score, arrs["q"], arrs["k"], arrs["v"], 1) == orc.ERANGE, (which, hex(val))
    # just below the bound in V: accepted, every score finite
    vb = v.copy()
    vb.reshape(-1)[5] = 0x577F
    s = orc.score(q, k, vb, 1)
    assert np.all(np.isfinite(s[:, :-2])) and s.max() > 1e20
    # in Q or K just below the bound: not ERANGE (this row's softmax is one-hot, so
    # it is rejected as singular instead)
    for which in ("q", "k"):
        arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
        arrs[which].reshape(-1)[5] = 0x577F
        assert _status(orc.score, arrs["q"], arrs["k"], arrs["v"], 1) in (orc.OK, orc.ESINGULAR)


def test_input_contract_precedence():
    """Non-finite before out-of-range before singular."""
    q, k, v = _tiny_inputs(2, 1, 1, d=8, n=10, w=2)
    a = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
    a["v"].reshape(-1)[3] = 0x7FC0     # NaN
    a["k"].reshape(-1)[4] = 0x5780     # 2^48
    assert _status(orc.score, a["q"], a["k"], a["v"], 1) == orc.ENONFINITE
    b = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
    b["q"].reshape(-1)[0] = 0x5780     # out of range, and one-hot rows (singular)
    assert _status(orc.score, b["q"], b["k"], b["v"], 1) == orc.ERANGE


def test_attention_scores_ignore_v_and_check_q_k():
    q, k, v = _tiny_inputs(2, 1, 1, d=8, n=10, w=2)
    for which in ("q", "k"):
        a = {"q": q.copy(), "k": k.copy()}
        a[which].reshape(-1)[2] = 0xD780
        assert _status(orc.attention_score, a["q"], a["k"], 1) == orc.ERANGE


def test_score_beyond_float32_is_erange():
    q, k, v = _tiny_inputs(2, 1, 1, d=8, n=10, w=2)
    v = wl.bf16_bits(wl.bf16_to_f32(v) * np.float32(1e36))
    with pytest.raises(orc.OracleError) as e:
        orc.score(q, k, v, pool=1)
    assert e.value.code == orc.ERANGE


# --- input generator: deterministic, and its stated structure is present
def test_generator_deterministic_and_structured():
    cfg = wl.custom(Hq=8, Hkv=2, d=64, n=256, w=4, pool=7, budget=32, seed=11, recipe="llama")
    a = wl.make_layer(cfg, cfg.seed)
    b = wl.make_layer(cfg, cfg.seed)
    c = wl.make_layer(cfg, cfg.seed + 1)
    assert wl.digest([a["q"], a["k"], a["v"]]) == wl.digest([b["q"], b["k"], b["v"]])
    assert wl.digest([a["q"], a["k"], a["v"]]) != wl.digest([c["q"], c["k"], c["v"]])
    qf, kf = brute.widen(a["q"]), brute.widen(a["k"])
    for g in range(2):
        std = kf[g, 4:].std(axis=0)
        assert (std > 4).sum() == 4                  # four outlier channels x8
        Qg = qf[g * 4:(g + 1) * 4].reshape(-1, 64)
        # sinks: every window query's logit on keys 0..3 is its ordinary N(0, ~1.7^2)
        # logit plus 6, so the mean over the group's queries and sinks sits near 6
        sink = (Qg @ kf[g, :4].T) / 8.0
        plain = (Qg @ kf[g, 4:].T) / 8.0
        assert abs(sink.mean() - 6.0) < 1.0 and abs(plain.mean()) < 0.5


def test_sink_heavy_recipe_puts_most_mass_on_token_0():
    """Every window query of the sink-heavy Llama case puts more than 0.94 of its
    attention on token 0 (plain float64 softmax over its visible keys)."""
    cfg = wl.CONFIGS["llama4k_sink"]
    inp = wl.make_layer(cfg, cfg.seed)
    qf, kf = brute.widen(inp["q"]), brute.widen(inp["k"])
    G, n, w, d = cfg.G, cfg.n, cfg.w, cfg.d
    for h in range(cfg.Hq):
        g = h // G
        for t in range(w):
            l = (kf[g, :n - w + t + 1] @ qf[h, t]) / np.sqrt(d)
            p = np.exp(l - l.max())
            p /= p.sum()
            assert int(np.argmax(p)) == 0 and p[0] > 0.94, (h, t, p[0])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, np.inf, -np.inf], dtype=np.float32)
    b = wl.bf16_bits(x)
    np.testing.assert_array_equal(b, np.array([0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F80, 0xFF80],
                                              dtype=np.uint16))
    t = torch.from_numpy(np.random.default_rng(0).standard_normal(1000).astype(np.float32))
    np.testing.assert_array_equal(wl.bf16_bits(t.numpy()),
                                  t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# --- regression fixture written by tests/golden/make_golden.py from the oracle alone
def test_tiny_golden_fixture_reproduces():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")))
    cfg = wl.TINY
    inp = wl.make_layer(cfg, cfg.seed, accept=lambda q, k, v: orc.max_probability(q, k, v) <= 0.5)
    assert inp["tries"] == g["tries"]
    assert wl.digest([inp["q"], inp["k"], inp["v"]]) == g["input_sha256"]
    raw = orc.raw_scores(inp["q"], inp["k"], inp["v"])
    np.testing.assert_allclose(raw, np.array(g["raw"]), rtol=1e-14)
    scores = orc.pool_protect(raw, cfg.w, cfg.pool)
    np.testing.assert_array_equal(orc.select(scores, cfg.budget), np.array(g["keep"], dtype=np.int32))


def test_thread_count_does_not_change_a_bit():
    """The oracle spreads a call over the window rows of every KV head and adds
    each head's rows in a fixed order: the scores are bitwise the same on one
    thread and on several."""
    rng = np.random.default_rng(8)
    q = wl.bf16_bits(rng.standard_normal((8, 3, 16), dtype=np.float32))
    k = wl.bf16_bits(rng.standard_normal((2, 300, 16), dtype=np.float32))
    v = wl.bf16_bits(rng.standard_normal((2, 300, 16), dtype=np.float32))
    one = orc.score(q, k, v, 5, nthreads=1)
    for t in (2, 3, 7):
        assert np.array_equal(one.view(np.uint64), orc.score(q, k, v, 5, nthreads=t).view(np.uint64))
