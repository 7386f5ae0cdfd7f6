"""Layer-wide selection (cross-head budgets) through the C ABI against the
oracle: bit-exact on identical scores; on the full path, eviction sets equal
outside the 2e-3 band around the layer's k-th smallest oracle score, and the
packed cache bit-exact."""
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


def _layer_select(ctx, s, budget):
    Hkv, n = s.shape
    sd = torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).cuda()
    gk = H.Guarded((max(budget, 1),), torch.int32, -9)
    gc = H.Guarded((Hkv,), torch.int32, -9)
    keep, counts = gk.t, gc.t
    ctx.select_layer(sd, Hkv, n, budget, keep, counts)
    st = ctx.sync()
    gk.check("keep")
    gc.check("counts")
    return st, keep.cpu().numpy()[:budget], counts.cpu().numpy()


@pytest.mark.parametrize("Hkv,n", [(1, 1), (3, 50), (8, 4097), (8, 131072), (64, 3000)])
def test_exact_on_identical_scores(ctx, Hkv, n):
    print(f"[case] layer select {Hkv}x{n}", flush=True)
    rng = np.random.default_rng(Hkv * 7 + n)
    s = rng.integers(0, 60, size=(Hkv, n)).astype(np.float32)      # heavy ties
    s[:, : n // 2] = rng.random((Hkv, n // 2)).astype(np.float32)
    s[:, -min(4, n):] = np.inf
    total = Hkv * n
    for budget in sorted({0, 1, min(total, 4 * Hkv), total // 2, total - 1, total}):
        st, keep, counts = _layer_select(ctx, s, budget)
        assert st == dropkv.OK
        want_keep, want_counts = orc.select_layer(s.astype(np.float64), budget)
        np.testing.assert_array_equal(keep, want_keep, err_msg=f"budget {budget}")
        np.testing.assert_array_equal(counts, want_counts, err_msg=f"budget {budget}")


def test_alternating_with_per_head_selection(ctx):
    """The per-head and layer-wide selections keep separate scratch."""
    rng = np.random.default_rng(5)
    s = rng.random((8, 5000)).astype(np.float32)
    sd = torch.from_numpy(s).cuda()
    for _ in range(3):
        keep = torch.empty((8, 300), dtype=torch.int32, device="cuda")
        ctx.select(sd, 8, 5000, 300, keep)
        assert ctx.sync() == dropkv.OK
        np.testing.assert_array_equal(keep.cpu().numpy(), orc.select(s.astype(np.float64), 300))
        st, kl, cl = _layer_select(ctx, s, 2400)
        assert st == dropkv.OK
        wk, wc = orc.select_layer(s.astype(np.float64), 2400)
        np.testing.assert_array_equal(kl, wk)
        np.testing.assert_array_equal(cl, wc)


def test_full_path_llama32k(ctx):
    """score -> layer-wide select (same total budget as the per-head one) ->
    packed cache, against the oracle."""
    cfg = wl.CONFIGS["llama32k"]
    inp = wl.make_layer(cfg, cfg.seed)
    q, k, v = inp["q"], inp["k"], inp["v"]
    Hkv, n, d = cfg.Hkv, cfg.n, cfg.d
    budget = Hkv * cfg.budget
    qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    outs = dict(scores=H.Guarded((Hkv, n), torch.float32), keep=H.Guarded((budget,), torch.int32),
                counts=H.Guarded((Hkv,), torch.int32), k_out=H.Guarded((budget, d), torch.int16),
                v_out=H.Guarded((budget, d), torch.int16))
    scores, keep, counts, ko, vo = (outs[x].t for x in ("scores", "keep", "counts", "k_out", "v_out"))
    ctx.score(qd, kd, vd, n, cfg.w, cfg.Hq, Hkv, d, cfg.pool, scores)
    ctx.select_layer(scores, Hkv, n, budget, keep, counts)
    ctx.compact(kd, vd, 1, Hkv * n, d, keep, budget, ko, vo)
    assert ctx.sync() == dropkv.OK
    for name, g in outs.items():
        g.check(name)
    want = orc.score(q, k, v, cfg.pool)
    kg, cg = keep.cpu().numpy(), counts.cpu().numpy()
    assert cg.sum() == budget and np.all(cg >= cfg.w)
    assert np.all(np.diff(kg) > 0)
    # eviction decisions equal outside the band around the layer threshold
    flat = want.reshape(-1)
    order = np.lexsort((np.arange(flat.size), flat))
    T = flat[order[flat.size - budget - 1]]
    band = np.abs(flat - T) <= 2e-3 * abs(T)
    ev_g = np.ones(flat.size, bool); ev_g[kg] = False
    wk, _ = orc.select_layer(want, budget)
    ev_o = np.ones(flat.size, bool); ev_o[wk] = False
    assert not ((ev_g != ev_o) & ~band).any()
    # the packed rows are the kept rows of the [Hkv][n][d] cache, bit for bit
    np.testing.assert_array_equal(ko.cpu().numpy().view(np.uint16), k.reshape(Hkv * n, d)[kg])
    np.testing.assert_array_equal(vo.cpu().numpy().view(np.uint16), v.reshape(Hkv * n, d)[kg])
