"""Attention-only (SnapKV-style) scores: the HIP path vs the float64 oracle,
element by element, through the C ABI (dropkv_score_attention).

Bar: |gpu - oracle| <= 2e-3 |oracle| + FLT_MIN per score, identical +inf
positions, eviction sets identical outside the 2e-3 band around the oracle's
k-th smallest score.
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


def _rand(seed, Hq, Hkv, d, n, w, qscale=1.0):
    rng = np.random.default_rng(seed)
    q = wl.bf16_bits((qscale * rng.standard_normal((Hq, w, d))).astype(np.float32))
    k = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    return q, k


def _gpu_attention(ctx, q, k, pool, budget=None):
    Hq, w, d = q.shape
    Hkv, n, _ = k.shape
    qd, kd = H.to_dev(q), H.to_dev(k)
    gs = H.Guarded((Hkv, n), torch.float32, -7.0)
    scores = gs.t
    ctx.score_attention(qd, kd, n, w, Hq, Hkv, d, pool, scores)
    keep = gk = None
    if budget:
        gk = H.Guarded((Hkv, budget), torch.int32, -5)
        keep = gk.t
        ctx.select(scores, Hkv, n, budget, keep)
    st = ctx.sync()
    torch.cuda.synchronize()
    gs.check("scores")
    if gk is not None:
        gk.check("keep")
    return st, scores.cpu().numpy(), (keep.cpu().numpy() if keep is not None else None)


def _check(ctx, q, k, pool, budget, where):
    print(f"[case] {where}", flush=True)
    st, s, keep = _gpu_attention(ctx, q, k, pool, budget)
    assert st == dropkv.OK, f"{where}: device status {st}"
    want = orc.attention_score(q, k, pool)
    H.assert_scores_close(s, want, where=where)
    if budget:
        H.assert_keep_sets_match(keep, orc.select(want, budget), want, budget, where=where)
    return s, want


def test_tiny_config(ctx):
    cfg = wl.TINY
    inp = wl.make_layer(cfg, cfg.seed)
    _check(ctx, inp["q"], inp["k"], cfg.pool, cfg.budget, "tiny")


SHAPES = [
    (1, 1, 8, 1, 1, 1),        # one visible key: p = 1 is fine here
    (2, 1, 8, 2, 1, 3),
    (2, 2, 64, 33, 1, 3),
    (8, 8, 96, 300, 4, 5),
    (32, 8, 128, 1000, 8, 7),
    (4, 1, 128, 2049, 8, 7),
    (8, 2, 40, 777, 2, 9),
    (2, 1, 256, 600, 4, 3),
    (16, 1, 128, 5000, 2, 31),
    (3, 1, 72, 1500, 5, 129),
    (1, 1, 16, 4096, 32, 3),
    (6, 2, 200, 1100, 7, 11),
    # G * w = 8 (one 8-row block: the reduced second-pass instance) and 9 (not)
    (4, 4, 96, 2500, 8, 7),      # Phi-3-mini-shaped heads: G = 1, w = 8
    (8, 4, 128, 1700, 4, 3),     # G = 2, w = 4
    (3, 3, 64, 900, 9, 5),       # G = 1, w = 9
    (28, 4, 128, 3000, 8, 7),    # 56 rows per KV head
    (9, 1, 40, 700, 5, 3),       # 45 rows
    (16, 1, 64, 1500, 8, 5),     # 128 rows
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(ctx, shape):
    Hq, Hkv, d, n, w, pool = shape
    q, k = _rand(hash(shape) % 10000 + 17, Hq, Hkv, d, n, w, qscale=2.0)
    _check(ctx, q, k, pool, max(w, n // 10), f"attention shape {shape}")


@pytest.mark.parametrize("name", ["llama4k", "llama32k", "llama128k"])
def test_llama_configs(ctx, name):
    cfg = wl.CONFIGS[name]
    inp = wl.make_layer(cfg, cfg.seed)
    _check(ctx, inp["q"], inp["k"], cfg.pool, cfg.budget, f"attention {name}")


def test_peaked_rows_are_not_errors(ctx):
    """A probability that rounds to 1 rejects DropKV scores but not attention sums."""
    n, d = 40, 8
    q = np.zeros((1, 1, d), np.float32); q[0, 0, 0] = 1.0
    k = np.zeros((1, n, d), np.float32); k[0, 5, 0] = 60.0 * np.sqrt(d)
    q, k = wl.bf16_bits(q), wl.bf16_bits(k)
    st, s, _ = _gpu_attention(ctx, q, k, 3)
    assert st == dropkv.OK
    H.assert_scores_close(s, orc.attention_score(q, k, 3), where="peaked")


def test_nonfinite_rejected(ctx):
    q, k = _rand(3, 4, 2, 16, 100, 3)
    k[1, 37, 5] = 0x7FC0   # NaN
    st, _, _ = _gpu_attention(ctx, q, k, 3)
    assert st == dropkv.ENONFINITE


@pytest.mark.parametrize("which", ["q", "k"])
def test_input_contract(ctx, which):
    """Reading R-11: a query or key element of magnitude >= 2^48 is ERANGE on both
    sides (the attention-only scores read no values)."""
    q, k = _rand(4, 4, 2, 16, 300, 3)
    arr = q if which == "q" else k
    arr.reshape(-1)[7 if which == "q" else 200 * 16 + 3] = 0xD780
    with pytest.raises(orc.OracleError) as e:
        orc.attention_score(q, k, 3)
    assert e.value.code == orc.ERANGE
    st, _, _ = _gpu_attention(ctx, q, k, 3)
    assert st == dropkv.ERANGE


def test_bitwise_deterministic(ctx):
    q, k = _rand(8, 32, 8, 128, 20000, 8)
    a = _gpu_attention(ctx, q, k, 7)[1]
    b = _gpu_attention(ctx, q, k, 7)[1]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_host_argument_checks(ctx):
    q, k = _rand(1, 4, 2, 16, 50, 3)
    qd, kd = H.to_dev(q), H.to_dev(k)
    s = torch.empty((2, 50), dtype=torch.float32, device="cuda")
    L = dropkv.lib()
    h = ctx._h
    P = lambda t: t.data_ptr()
    assert L.dropkv_score_attention(h, P(qd), P(kd), 50, 3, 4, 2, 16, 4, P(s), None) == dropkv.EINVAL  # even pool
    assert L.dropkv_score_attention(h, P(qd), P(kd), 50, 3, 4, 3, 16, 3, P(s), None) == dropkv.EINVAL  # Hq % Hkv
    assert L.dropkv_score_attention(h, P(qd), None, 50, 3, 4, 2, 16, 3, P(s), None) == dropkv.EINVAL
    assert L.dropkv_score_attention(h, P(qd), P(kd), 50, 60, 4, 2, 16, 3, P(s), None) == dropkv.EINVAL  # w > n
    assert ctx.sync() == dropkv.OK
