"""dropkv_score_ex: the window queries' attention outputs and log-sum-exps
handed back by the first pass, against the float64 oracle.

Bar: per window query, |a_gpu - a_oracle| <= 2e-3 * max_i |a_oracle[i]| for
every element; |lse_gpu - lse_oracle| <= 1e-4 * max(1, |lse_oracle|).  The
scores are bitwise those of dropkv_score.
"""
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


def _rand(seed, Hq, Hkv, d, n, w):
    rng = np.random.default_rng(seed)
    q = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    k = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    v = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    return q, k, v


def _run(ctx, q, k, v, pool):
    Hq, w, d = q.shape
    Hkv, n, _ = k.shape
    qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    outs = dict(s1=H.Guarded((Hkv, n), torch.float32), s2=H.Guarded((Hkv, n), torch.float32),
                out_a=H.Guarded((Hq, w, d), torch.float32, 7.0),
                out_lse=H.Guarded((Hq, w), torch.float32, 7.0))
    s1, s2, oa, ol = (outs[x].t for x in ("s1", "s2", "out_a", "out_lse"))
    ctx.score(qd, kd, vd, n, w, Hq, Hkv, d, pool, s1)
    ctx.score_ex(qd, kd, vd, n, w, Hq, Hkv, d, pool, s2, oa, ol)
    st = ctx.sync()
    for name, g in outs.items():
        g.check(name)
    return st, s1.cpu().numpy(), s2.cpu().numpy(), oa.cpu().numpy(), ol.cpu().numpy()


CASES = [("tiny", None), ("shape", (8, 2, 40, 777, 2, 9)), ("shape", (32, 8, 128, 3000, 8, 7)),
         ("shape", (4, 1, 256, 700, 5, 3)), ("shape", (28, 4, 128, 1000, 8, 7)),
         ("shape", (9, 1, 40, 700, 5, 3)), ("llama4k", None)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0] if c[1] is None else "x".join(map(str, c[1])))
def test_window_outputs_match_oracle(ctx, case):
    name, shape = case
    print(f"[case] window outputs {case}", flush=True)
    if name == "shape":
        Hq, Hkv, d, n, w, pool = shape
        q, k, v = _rand(hash(shape) % 1000, Hq, Hkv, d, n, w)
    else:
        cfg = wl.CONFIGS[name] if name != "tiny" else wl.TINY
        inp = wl.make_layer(cfg, cfg.seed)
        q, k, v, pool = inp["q"], inp["k"], inp["v"], cfg.pool
    st, s1, s2, oa, ol = _run(ctx, q, k, v, pool)
    assert st == dropkv.OK
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32)), "score_ex changed the scores"
    _, a_want, _ = orc.window_attention(q, k, v)
    lse_want = orc.window_lse(q, k)
    scale = np.abs(a_want).max(axis=2, keepdims=True)
    err = np.abs(oa.astype(np.float64) - a_want)
    assert np.all(err <= 2e-3 * scale + 1e-30), f"a: worst {float((err / (scale + 1e-30)).max()):.3e}"
    lerr = np.abs(ol.astype(np.float64) - lse_want)
    assert np.all(lerr <= 1e-4 * np.maximum(1.0, np.abs(lse_want))), f"lse: worst {float(lerr.max()):.3e}"


def test_null_outputs_are_allowed(ctx):
    q, k, v = _rand(3, 4, 2, 16, 100, 3)
    qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    s = torch.empty((2, 100), dtype=torch.float32, device="cuda")
    ctx.score_ex(qd, kd, vd, 100, 3, 4, 2, 16, 3, s)
    assert ctx.sync() == dropkv.OK
