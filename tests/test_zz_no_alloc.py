"""dropkv_score_noalloc (the entry point for callers that cannot allocate) through
the C ABI against dropkv_score, on calls in a row -- the second with a smaller
input, the third sink-heavy (every row takes the exact fixup, whose arrival
counters then sit where the earlier layouts kept partial sums) -- plus the size
limit of its static scratch.  The scores must be the same bits: both run the
same kernels on the same inputs."""
import ctypes

import numpy as np
import pytest
import torch

from attention_perturbation_scoring_amd import dropkv, workload as wl
from oracle import oracle as orc
import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _noalloc(ctx, qd, kd, vd, n, w, Hq, Hkv, d, pool, scores):
    L = dropkv.lib()
    return L.dropkv_score_noalloc(ctx._h, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), n, w, Hq,
                                  Hkv, d, pool, scores.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)


def _inputs(seed, Hq, Hkv, d, n, w):
    rng = np.random.default_rng(seed)
    q = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    k = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    v = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    return q, k, v


def test_noalloc_matches_score_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = wl.LLAMA_32K
    big = wl.make_layer(cfg, cfg.seed)
    sink_cfg = wl.LLAMA_4K_SINK
    sink = wl.make_layer(sink_cfg, sink_cfg.seed)
    cases = [((big["q"], big["k"], big["v"]), (cfg.n, cfg.w, cfg.Hq, cfg.Hkv, cfg.d, cfg.pool)),
             (_inputs(5, 8, 2, 96, 3001, 4), (3001, 4, 8, 2, 96, 5)),   # smaller, ragged
             ((sink["q"], sink["k"], sink["v"]),
              (sink_cfg.n, sink_cfg.w, sink_cfg.Hq, sink_cfg.Hkv, sink_cfg.d, sink_cfg.pool))]
    with dropkv.Context(0) as ref, dropkv.Context(0) as ctx:
        for (q, k, v), (n, w, Hq, Hkv, d, pool) in cases:
            print(f"[case] noalloc n={n} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
            qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
            want = H.Guarded((Hkv, n), torch.float32, -1.0)
            got = H.Guarded((Hkv, n), torch.float32, -2.0)
            ref.score(qd, kd, vd, n, w, Hq, Hkv, d, pool, want.t)
            assert ref.sync() == dropkv.OK
            torch.cuda.synchronize()
            free0 = torch.cuda.mem_get_info()[0]
            assert _noalloc(ctx, qd, kd, vd, n, w, Hq, Hkv, d, pool, got.t) == dropkv.OK
            assert ctx.sync() == dropkv.OK
            torch.cuda.synchronize()
            # a fresh context's dropkv_score would have allocated its scratch here
            assert torch.cuda.mem_get_info()[0] >= free0 - (1 << 20)
            got.check("noalloc scores")
            np.testing.assert_array_equal(got.t.cpu().numpy().view(np.uint32),
                                          want.t.cpu().numpy().view(np.uint32))
            if n == 3001:   # the smaller case also against the oracle (the same bar as every score)
                H.assert_scores_close(got.t.cpu().numpy(), orc.score(q, k, v, pool), where="noalloc small")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    limit = dropkv.lib().dropkv_noalloc_scratch_bytes()
    # 1024 folded heads of d = 96 need about 39 MB of split states
    n, w, Hq, Hkv, d = 131072, 8, 1024, 1024, 96
    need, _ = dropkv.scratch_bytes(n, w, Hq, Hkv, d)
    assert need > limit
    small = torch.zeros(64, dtype=torch.int16, device="cuda")   # never read: rejected first
    sc = torch.zeros(64, dtype=torch.float32, device="cuda")
    with dropkv.Context(0) as ctx:
        assert _noalloc(ctx, small, small, small, n, w, Hq, Hkv, d, 7, sc) == dropkv.ESCRATCH
        assert ctx.sync() == dropkv.OK
