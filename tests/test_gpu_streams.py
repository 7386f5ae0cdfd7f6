"""The C ABI on a caller's non-default stream.

PyTorch creates its side streams non-blocking: they do not wait for work on the
null stream.  Every call of a fresh context (first scratch allocation and
zeroing, later re-layouts when the head count changes) must still be ordered on
the caller's stream, and give the same bits as on the default stream.
"""
import numpy as np
import pytest
import torch

from attention_perturbation_scoring_amd import dropkv, workload as wl
from oracle import oracle as orc
import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _rand(seed, Hq, Hkv, d, n, w):
    rng = np.random.default_rng(seed)
    q = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    k = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    v = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    return q, k, v


def _path_on(stream, q, k, v, pool, budget):
    ctx = dropkv.Context(0)   # fresh: its scratch is allocated and zeroed by these calls
    try:
        with torch.cuda.stream(stream):
            return H.gpu_path(ctx, q, k, v, pool, budget)
    finally:
        ctx.close()


@pytest.mark.parametrize("case", ["llama4k", "rows56"])
def test_fresh_context_on_side_stream_matches_default_stream(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if case == "llama4k":
        cfg = wl.CONFIGS["llama4k"]
        inp = wl.make_layer(cfg, cfg.seed)
        q, k, v, pool, budget = inp["q"], inp["k"], inp["v"], cfg.pool, cfg.budget
    else:   # G = 7, w = 8: two row groups per KV head
        q, k, v = _rand(31, 28, 4, 128, 3000, 8)
        pool, budget = 7, 300
    print(f"[case] side stream {case}", flush=True)
    side = torch.cuda.Stream()
    got = _path_on(side, q, k, v, pool, budget)
    ref = _path_on(torch.cuda.default_stream(), q, k, v, pool, budget)
    assert got[0] == dropkv.OK and ref[0] == dropkv.OK
    for a, b, what in zip(got[1:], ref[1:], ("scores", "keep", "k_out", "v_out")):
        np.testing.assert_array_equal(a, b, err_msg=f"{case}: {what} differ between streams")
    want = orc.score(q, k, v, pool)
    H.assert_scores_close(got[1], want, where=f"{case} side stream")
    H.assert_keep_sets_match(got[2], orc.select(want, budget), want, budget,
                             where=f"{case} side stream")


def test_selection_relayout_on_side_stream():
    """A context's selection scratch is re-laid out (and its counters zeroed)
    when the head count changes; on a side stream the zeroing must precede the
    kernel that relies on it."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(5)
    side = torch.cuda.Stream()
    ctx = dropkv.Context(0)
    try:
        with torch.cuda.stream(side):
            for Hkv, n, budget in ((8, 40000, 2000), (3, 70000, 5000), (8, 40000, 2000)):
                print(f"[case] side-stream select Hkv={Hkv} n={n}", flush=True)
                s = rng.integers(0, 1000, size=(Hkv, n)).astype(np.float32)
                s[:, -4:] = np.inf
                sd = torch.from_numpy(s).cuda()
                keep = torch.full((Hkv, budget), -3, dtype=torch.int32, device="cuda")
                ctx.select(sd, Hkv, n, budget, keep)
                assert ctx.sync() == dropkv.OK
                np.testing.assert_array_equal(keep.cpu().numpy(),
                                              orc.select(s.astype(np.float64), budget),
                                              err_msg=f"Hkv={Hkv} n={n}")
    finally:
        ctx.close()
