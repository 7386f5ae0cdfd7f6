"""dropkv_score_select (scoring with the selection's first radix digit counted
in the second pass, then the selection) against dropkv_score + dropkv_select:
the same score bits and the same keep list, on heads large enough for the
single-launch team selection that starts from that histogram and on sizes that
fall back to the two calls; and a withheld selection (latched error) leaves
the histogram scratch clean for the calls after it."""
import numpy as np
import pytest
import torch

from attention_perturbation_scoring_amd import dropkv, workload as wl
from oracle import oracle as orc
import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = dropkv.Context(0)
    yield c
    c.close()


def _both(ctx, q, k, v, n, w, Hq, Hkv, d, pool, budget):
    qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    s1 = H.Guarded((Hkv, n), torch.float32, -1.0)
    s2 = H.Guarded((Hkv, n), torch.float32, -2.0)
    k1 = H.Guarded((Hkv, max(budget, 1)), torch.int32, -3)
    k2 = H.Guarded((Hkv, max(budget, 1)), torch.int32, -4)
    ctx.score(qd, kd, vd, n, w, Hq, Hkv, d, pool, s1.t)
    if budget:
        ctx.select(s1.t, Hkv, n, budget, k1.t)
    st1 = ctx.sync()
    ctx.score_select(qd, kd, vd, n, w, Hq, Hkv, d, pool, budget, s2.t, k2.t)
    st2 = ctx.sync()
    for g_ in (s1, s2, k1, k2):
        g_.check("score_select outputs")
    return st1, st2, s1.t.cpu().numpy(), s2.t.cpu().numpy(), k1.t.cpu().numpy(), k2.t.cpu().numpy()


def _same(ctx, q, k, v, n, w, Hq, Hkv, d, pool, budget, where):
    print(f"[case] {where}", flush=True)
    st1, st2, s1, s2, k1, k2 = _both(ctx, q, k, v, n, w, Hq, Hkv, d, pool, budget)
    assert st1 == dropkv.OK and st2 == dropkv.OK, f"{where}: status {st1} / {st2}"
    np.testing.assert_array_equal(s2.view(np.uint32), s1.view(np.uint32), err_msg=where)
    if budget:
        np.testing.assert_array_equal(k2[:, :budget], k1[:, :budget], err_msg=where)
    return s2, k2


@pytest.mark.parametrize("name", ["llama32k", "llama128k", "llama128k_sink"])
def test_prebuilt_histogram_path_matches_the_two_calls(ctx, name):
    cfg = wl.CONFIGS[name]
    inp = wl.make_layer(cfg, cfg.seed)
    for budget in (cfg.budget, cfg.n // 2, cfg.w):
        s, keep = _same(ctx, inp["q"], inp["k"], inp["v"], cfg.n, cfg.w, cfg.Hq, cfg.Hkv, cfg.d,
                        cfg.pool, budget, f"{name} budget {budget}")
        # the survivors are exactly those of the (score, index) order on these scores
        want = orc.select(s.astype(np.float64), budget)
        np.testing.assert_array_equal(keep[:, :budget], want)


@pytest.mark.parametrize("n,budget", [(3001, 300), (16384, 1000), (20000, 0), (20000, 20000)])
def test_other_sizes_match_the_two_calls(ctx, n, budget):
    Hq, Hkv, d, w, pool = 8, 2, 128, 8, 7
    rng = np.random.default_rng(n + budget)
    q = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    k = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    v = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    _same(ctx, q, k, v, n, w, Hq, Hkv, d, pool, budget, f"n={n} budget={budget}")


def test_withheld_selection_leaves_the_histogram_clean(ctx):
    cfg = wl.CONFIGS["llama32k"]
    inp = wl.make_layer(cfg, cfg.seed)
    bad_k = inp["k"].copy()
    bad_k[1, 1234, 5] = 0x7FC0   # a NaN key: the call is rejected, no keep list
    Hq, Hkv, d, n, w, pool, budget = cfg.Hq, cfg.Hkv, cfg.d, cfg.n, cfg.w, cfg.pool, cfg.budget
    qd, kd, vd = H.to_dev(inp["q"]), H.to_dev(bad_k), H.to_dev(inp["v"])
    sc = torch.empty((Hkv, n), dtype=torch.float32, device="cuda")
    keep = H.Guarded((Hkv, budget), torch.int32, -9)
    print("[case] score_select on a rejected input", flush=True)
    ctx.score_select(qd, kd, vd, n, w, Hq, Hkv, d, pool, budget, sc, keep.t)
    assert ctx.sync() == dropkv.ENONFINITE
    assert bool((keep.t == -9).all()), "a keep list was written for a rejected call"
    keep.check("withheld keep")
    # the next calls see a clean histogram: same results as the two calls
    for i in range(2):
        _same(ctx, inp["q"], inp["k"], inp["v"], n, w, Hq, Hkv, d, pool, budget,
              f"after the rejected call, call {i}")


def test_alternating_parities_and_paths(ctx):
    """The single-launch selection keeps its histograms and counters in two
    sets, used by calls of alternating parity (each call clears the other set
    for the next): an uneven mix of prebuilt-histogram calls and plain
    selections meets both sets from both paths, and every call stays exact."""
    cfg = wl.CONFIGS["llama32k"]
    inp = wl.make_layer(cfg, cfg.seed)
    n, Hkv, B = cfg.n, cfg.Hkv, cfg.budget
    qd, kd, vd = H.to_dev(inp["q"]), H.to_dev(inp["k"]), H.to_dev(inp["v"])
    s = torch.empty((Hkv, n), dtype=torch.float32, device="cuda")
    ctx.score(qd, kd, vd, n, cfg.w, cfg.Hq, Hkv, cfg.d, cfg.pool, s)
    assert ctx.sync() == dropkv.OK
    want = orc.select(s.cpu().numpy().astype(np.float64), B)
    keep = H.Guarded((Hkv, B), torch.int32, -5)
    for i, kind in enumerate(["ss", "sel", "sel", "ss", "ss", "sel", "ss", "sel"]):
        print(f"[case] call {i}: {kind}", flush=True)
        keep.t.fill_(-1)
        if kind == "ss":
            ctx.score_select(qd, kd, vd, n, cfg.w, cfg.Hq, Hkv, cfg.d, cfg.pool, B, s, keep.t)
        else:
            ctx.select(s, Hkv, n, B, keep.t)
        assert ctx.sync() == dropkv.OK, f"call {i} ({kind})"
        keep.check(f"call {i}")
        np.testing.assert_array_equal(keep.t.cpu().numpy(), want, err_msg=f"call {i} ({kind})")


@pytest.mark.parametrize("case", range(10))
def test_seeded_shapes_match_the_two_calls(ctx, case):
    """A seeded sweep over what the one-call path depends on: team sizes 2..8
    (ragged last members), 1..8 KV heads, d 64..256, one to three 32-row groups
    per KV head (G * w up to 96) and budgets anywhere in (0, n); every case is
    bitwise the two calls, and the keep list is the oracle's selection on the
    same scores."""
    rng = np.random.default_rng(1000 + case)
    n = int(rng.integers(16385, 131073))
    Hkv = int(rng.choice([1, 2, 3, 8]))
    d = int(rng.choice([64, 96, 128, 256]))
    G = int(rng.choice([1, 2, 4, 12]))
    w = int(rng.choice([4, 8]))
    if d > 128 and G * w > 64:   # the wide-head layouts hold up to 96 window rows
        G = 8
    pool = int(rng.choice([1, 3, 7]))
    budget = int(rng.integers(w, n))
    Hq = G * Hkv
    q = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    k = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    v = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    where = f"case {case}: n={n} Hkv={Hkv} d={d} G={G} w={w} pool={pool} budget={budget}"
    s, keep = _same(ctx, q, k, v, n, w, Hq, Hkv, d, pool, budget, where)
    want = orc.select(s.astype(np.float64), budget)
    np.testing.assert_array_equal(keep[:, :budget], want, err_msg=where)
