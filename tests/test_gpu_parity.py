"""HIP path vs the float64 oracle, element by element, through the C ABI.

Bar (per score): |gpu - oracle| <= 2e-3 |oracle| + FLT_MIN, identical +inf
positions; eviction sets identical outside the 2e-3 band around the oracle's
k-th smallest score; compaction bit-exact; selection on identical scores exact.
"""
import math

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


def _rand(seed, Hq, Hkv, d, n, w, kscale=1.0):
    rng = np.random.default_rng(seed)
    q = wl.bf16_bits(rng.standard_normal((Hq, w, d), dtype=np.float32))
    k = wl.bf16_bits((kscale * rng.standard_normal((Hkv, n, d))).astype(np.float32))
    v = wl.bf16_bits(rng.standard_normal((Hkv, n, d), dtype=np.float32))
    return q, k, v


def _full_check(ctx, q, k, v, pool, budget, where):
    print(f"[case] {where}", flush=True)
    st, s, keep, ko, vo = H.gpu_path(ctx, q, k, v, pool, budget)
    try:
        want = orc.score(q, k, v, pool)
    except orc.OracleError as e:
        # the oracle rejects the input: the device must reach the same decision
        assert st == e.code, f"{where}: oracle status {e.code}, device status {st}"
        return None
    assert st == dropkv.OK, f"{where}: device status {st}"
    H.assert_scores_close(s, want, where=where)
    keep_o = orc.select(want, budget)
    H.assert_keep_sets_match(keep, keep_o, want, budget, where=where)
    # compaction is bit-exact for the GPU's own keep list
    np.testing.assert_array_equal(ko, orc.compact(k, keep))
    np.testing.assert_array_equal(vo, orc.compact(v, keep))
    return s, want, keep, keep_o


def test_tiny_config(ctx):
    cfg = wl.TINY
    inp = wl.make_layer(cfg, cfg.seed, accept=lambda q, k, v: orc.max_probability(q, k, v) <= 0.5)
    s, want, keep, keep_o = _full_check(ctx, inp["q"], inp["k"], inp["v"], cfg.pool, cfg.budget, "tiny")
    np.testing.assert_array_equal(keep, keep_o)


# (Hq, Hkv, d, n, w, pool): tiles, ragged tails, chunk halos, every d padding
SHAPES = [
    (1, 1, 8, 1, 1, 1),        # one visible key: p = 1, rejected as singular by both sides
    (2, 1, 8, 2, 1, 3),
    (2, 2, 64, 33, 1, 3),
    (8, 8, 96, 300, 4, 5),
    (32, 8, 128, 1000, 8, 7),
    (4, 1, 128, 2049, 8, 7),
    (8, 2, 40, 777, 2, 9),
    (2, 1, 256, 600, 4, 3),
    (16, 1, 128, 5000, 2, 31),
    (32, 32, 96, 3000, 1, 7),
    (3, 1, 72, 1500, 5, 129),
    (1, 1, 16, 4096, 32, 3),
    (6, 2, 200, 1100, 7, 11),
    # G * w = 8 (one 8-row block: the reduced second-pass instance) and 9 (not)
    (4, 4, 96, 2500, 8, 7),      # Phi-3-mini-shaped heads: G = 1, w = 8
    (8, 4, 128, 1700, 4, 3),     # G = 2, w = 4
    (3, 3, 64, 900, 9, 5),       # G = 1, w = 9
    # more than 32 window rows per KV head: row groups of 32
    (28, 4, 128, 3000, 8, 7),    # G = 7, w = 8: 56 rows (Qwen2.5-7B-shaped)
    (64, 8, 128, 2000, 8, 7),    # 64 rows, two full groups
    (9, 1, 40, 700, 5, 3),       # 45 rows, w does not divide 32
    (33, 1, 32, 300, 1, 3),      # 33 rows: one row in the second group
    (16, 1, 64, 1500, 8, 5),     # 128 rows, four groups
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(ctx, shape):
    Hq, Hkv, d, n, w, pool = shape
    q, k, v = _rand(hash(shape) % 10000, Hq, Hkv, d, n, w)
    budget = max(w, n // 10)
    _full_check(ctx, q, k, v, pool, budget, f"shape {shape}")


@pytest.mark.parametrize("name", ["llama4k", "llama32k", "llama128k", "llama4k_sink", "llama128k_sink"])
def test_llama_configs(ctx, name):
    cfg = wl.CONFIGS[name]
    inp = wl.make_layer(cfg, cfg.seed)
    s, want, keep, keep_o = _full_check(ctx, inp["q"], inp["k"], inp["v"], cfg.pool, cfg.budget, name)
    # the protected window survives
    for g in range(cfg.Hkv):
        assert set(range(cfg.n - cfg.w, cfg.n)) <= set(keep[g].tolist())


def test_select_exact_on_oracle_scores(ctx):
    """dropkv_select on the oracle's (fp32-rounded) scores gives the oracle's keep list."""
    rng = np.random.default_rng(3)
    # one-workgroup heads (n <= 16384, the last two at and just below the
    # limit) and a team of five (70000)
    for n, Hkv in ((1, 1), (50, 3), (4097, 2), (16384, 2), (16383, 3), (70000, 2)):
        s = rng.integers(0, 40, size=(Hkv, n)).astype(np.float32)      # heavy ties
        s[:, : n // 3] = rng.random((Hkv, n // 3)).astype(np.float32)
        s[:, -min(4, n):] = np.inf
        if n > 10:
            s[0, 5] = -0.0
            s[0, 6] = 0.0
        sd = torch.from_numpy(s).cuda()
        for budget in sorted({0, min(4, n), n // 2, n - 1, n} - {-1}):
            if budget < 0:
                continue
            keep = torch.full((Hkv, max(budget, 1)), -9, dtype=torch.int32, device="cuda")
            ctx.select(sd, Hkv, n, budget, keep)
            assert ctx.sync() == dropkv.OK
            if budget == 0:
                assert int(keep[0, 0]) == -9
                continue
            got = keep.cpu().numpy()[:, :budget]
            want = orc.select(s.astype(np.float64), budget)
            np.testing.assert_array_equal(got, want, err_msg=f"n={n} budget={budget}")


@pytest.mark.parametrize("n", [20000, 5000])
@pytest.mark.parametrize("kind", ["all_zero", "all_equal", "two_values", "negatives"])
def test_select_heavy_ties_and_signs(ctx, kind, n):
    """Threshold bins holding more than the candidate buffer, and negative keys;
    a team of two workgroups (20000) and one workgroup (5000) per head."""
    Hkv = 2
    rng = np.random.default_rng(11)
    if kind == "all_zero":
        s = np.zeros((Hkv, n), np.float32)
    elif kind == "all_equal":
        s = np.full((Hkv, n), 3.25, np.float32)
    elif kind == "two_values":
        s = np.where(rng.random((Hkv, n)) < 0.5, 1.0, 2.0).astype(np.float32)
    else:
        s = (rng.standard_normal((Hkv, n)) * 100).astype(np.float32)
        s[0, :50] = -0.0
    s[:, -8:] = np.inf
    sd = torch.from_numpy(s).cuda()
    for budget in (8, 100, n // 2 - 1, n - 1):
        keep = torch.full((Hkv, budget), -9, dtype=torch.int32, device="cuda")
        ctx.select(sd, Hkv, n, budget, keep)
        assert ctx.sync() == dropkv.OK
        np.testing.assert_array_equal(keep.cpu().numpy(), orc.select(s.astype(np.float64), budget),
                                      err_msg=f"{kind} n={n} budget={budget}")


def test_select_multi_launch_path(ctx):
    """Heads of two workgroups each, more workgroups than the device holds at
    once (2800 > 256 CUs x at most 10): selection runs as the multi-launch path
    instead of one launch, same result."""
    Hkv, n = 1400, 16500
    rng = np.random.default_rng(21)
    s = rng.integers(0, 300, size=(Hkv, n)).astype(np.float32)
    s[:, : n // 2] += rng.random((Hkv, n // 2)).astype(np.float32)
    s[:, -8:] = np.inf
    sd = torch.from_numpy(s).cuda()
    for budget in (8, 1000, n - 1):
        keep = torch.full((Hkv, budget), -9, dtype=torch.int32, device="cuda")
        ctx.select(sd, Hkv, n, budget, keep)
        assert ctx.sync() == dropkv.OK
        np.testing.assert_array_equal(keep.cpu().numpy(), orc.select(s.astype(np.float64), budget),
                                      err_msg=f"budget={budget}")


@pytest.mark.parametrize("wait", [-1, 0])
def test_select_when_teammates_do_not_arrive(ctx, wait):
    """A selection workgroup that stops waiting for its team finishes its share
    alone from the scores in memory: with every workgroup going alone (-1), or
    each going alone as soon as one poll finds a teammate missing (0; a mix
    of both paths), the keep lists equal the oracle's.  Heads of one to
    nine workgroups, heavy ties, a threshold bin larger than the candidate
    exchange, and the layer-wide selection."""
    rng = np.random.default_rng(40 + wait)
    try:
        ctx.set_select_wait(wait)
        for n, Hkv in ((20000, 3), (70000, 2), (131072, 8)):
            s = rng.integers(0, 50, size=(Hkv, n)).astype(np.float32)
            s[:, : n // 3] = rng.random((Hkv, n // 3)).astype(np.float32)
            s[:, -8:] = np.inf
            s[-1, : n // 2] = 2.5                                       # one huge threshold bin
            sd = torch.from_numpy(s).cuda()
            for budget in (8, n // 20, n // 2, n - 1):
                g = H.Guarded((Hkv, budget), torch.int32, -9)
                ctx.select(sd, Hkv, n, budget, g.t)
                assert ctx.sync() == dropkv.OK
                g.check("keep")
                np.testing.assert_array_equal(g.t.cpu().numpy(),
                                              orc.select(s.astype(np.float64), budget),
                                              err_msg=f"wait={wait} n={n} budget={budget}")
            total = Hkv * n
            gk = H.Guarded((total // 10,), torch.int32, -9)
            gc = H.Guarded((Hkv,), torch.int32, -9)
            ctx.select_layer(sd, Hkv, n, total // 10, gk.t, gc.t)
            assert ctx.sync() == dropkv.OK
            wk, wc = orc.select_layer(s.astype(np.float64), total // 10)
            np.testing.assert_array_equal(gk.t.cpu().numpy(), wk)
            np.testing.assert_array_equal(gc.t.cpu().numpy(), wc)
    finally:
        ctx.set_select_wait(16384)
    # the default afterwards: the team path, same answers
    s = rng.random((8, 131072)).astype(np.float32)
    keep = torch.empty((8, 6553), dtype=torch.int32, device="cuda")
    ctx.select(torch.from_numpy(s).cuda(), 8, 131072, 6553, keep)
    assert ctx.sync() == dropkv.OK
    np.testing.assert_array_equal(keep.cpu().numpy(), orc.select(s.astype(np.float64), 6553))


def test_singular_rejected_and_select_withheld(ctx):
    n, d = 40, 8
    q = np.zeros((1, 1, d), np.float32); q[0, 0, 0] = 1.0
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, n, d)).astype(np.float32); k[0, :, 0] = 0.0
    k[0, 7, 0] = 60.0 * math.sqrt(d)               # logit gap 60: S_excl ~ 1e-25 << 2^-53
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    q, k, v = wl.bf16_bits(q), wl.bf16_bits(k), wl.bf16_bits(v)
    with pytest.raises(orc.OracleError) as e:
        orc.score(q, k, v, 3)
    assert e.value.code == orc.ESINGULAR
    st, s, keep, _, _ = H.gpu_path(ctx, q, k, v, 3, 10, compact=False)
    assert st == dropkv.ESINGULAR
    assert np.all(keep == -5), "select must not write a keep list while an error is latched"
    # the latch is cleared by sync: a following good call succeeds
    q2, k2, v2 = _rand(2, 1, 1, d, n, 1)
    st, *_ = H.gpu_path(ctx, q2, k2, v2, 3, 10)
    assert st == dropkv.OK


@pytest.mark.parametrize("pstar", [0.9, 0.999, 1 - 1e-9])
@pytest.mark.parametrize("n,d", [(12, 8), (3000, 8), (3000, 96), (3000, 128), (1500, 256),
                                 (70000, 128)])
def test_near_singular_rows_match(ctx, pstar, n, d):
    """Rows whose arg-max holds most of the mass are accepted and match (the
    arg-max term goes through the exact exclusion path above p* ~ 0.94: one
    16-byte chunk per lane for d <= 128, two at d = 256; a long head at 70000)."""
    L = math.log(pstar * (n - 1) / (1 - pstar))
    rng = np.random.default_rng(5)
    q = np.zeros((2, 1, d), np.float32); q[:, 0, 0] = 1.0
    k = np.zeros((1, n, d), np.float32); k[0, :, 1:] = rng.standard_normal((n, d - 1))
    k[0, n // 3, 0] = L * math.sqrt(d)
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    q, k, v = wl.bf16_bits(q), wl.bf16_bits(k), wl.bf16_bits(v)
    _full_check(ctx, q, k, v, 1, max(1, n // 4), f"p*={pstar} n={n} d={d}")


def test_near_singular_heads_of_every_kind(ctx):
    """Four KV heads, four row groups each (G = 16, w = 8), every row peaked on
    one key placed differently per head: the first tile (p* = 0.999), inside
    the window so that rows t < 3 do not see it (p* = 0.95 for the rest), mid
    head below the fixup threshold (p* = 0.5), and the ragged last tile
    (p* = 1 - 1e-7).  Only the split holding the arg-max is streamed again for
    the fixed rows; the result must still be the exact exclusion."""
    Hq, Hkv, d, w, n = 64, 4, 128, 8, 20011
    rng = np.random.default_rng(17)
    q = np.zeros((Hq, w, d), np.float32); q[:, :, 0] = 1.0
    k = np.zeros((Hkv, n, d), np.float32); k[:, :, 1:] = rng.standard_normal((Hkv, n, d - 1))
    v = rng.standard_normal((Hkv, n, d)).astype(np.float32)
    for g, (pstar, j) in enumerate([(0.999, 7), (0.95, n - w + 3), (0.5, n // 2),
                                    (1 - 1e-7, n - 10)]):
        k[g, j, 0] = math.log(pstar * (n - 1) / (1 - pstar)) * math.sqrt(d)
    q, k, v = wl.bf16_bits(q), wl.bf16_bits(k), wl.bf16_bits(v)
    s, *_ = _full_check(ctx, q, k, v, 7, n // 4, "peaked heads G=16 w=8 n=20011")
    # the fixup's sums have a fixed order too: a second call gives the same bits
    again = H.gpu_path(ctx, q, k, v, 7, n // 4)
    np.testing.assert_array_equal(s.view(np.uint32), again[1].view(np.uint32))


def _peaked_with_copies(seed, Hq, Hkv, d, n, w, pstar, jstar, copies, near=(), near_scale=1e-2):
    """Every window row puts probability pstar on key jstar (logit gap from its
    key's first channel); the value rows at `copies` are exact copies of
    v_jstar (identical tokens have identical value rows) and those at `near`
    are v_jstar plus near_scale * N(0, 1) before the bf16 cast."""
    rng = np.random.default_rng(seed)
    q = np.zeros((Hq, w, d), np.float32); q[:, :, 0] = 1.0
    k = np.zeros((Hkv, n, d), np.float32); k[:, :, 1:] = rng.standard_normal((Hkv, n, d - 1))
    k[:, jstar, 0] = math.log(pstar * (n - 1) / (1 - pstar)) * math.sqrt(d)
    v = rng.standard_normal((Hkv, n, d)).astype(np.float32)
    v = wl.bf16_to_f32(wl.bf16_bits(v))
    for j in copies:
        v[:, j] = v[:, jstar]
    for j in near:
        v[:, j] = v[:, jstar] + near_scale * rng.standard_normal((Hkv, d)).astype(np.float32)
    return wl.bf16_bits(q), wl.bf16_bits(k), wl.bf16_bits(v)


@pytest.mark.parametrize("pstar", [0.99, 0.999, 0.9999])
@pytest.mark.parametrize("d", [96, 128, 256])
def test_value_rows_copying_the_argmax(ctx, pstar, d):
    """Tokens whose value row copies the dominant token's, one of them inside
    the window, and near copies: for them a - v is tiny next to ||a|| and ||v||,
    the expansion ||a||^2 - 2 a.v + ||v||^2 would cancel, and the distance must
    come out of the exact difference (notes, "Core equation": Delta_j =
    p_j/(1 - p_j) (a - v_j) for every token)."""
    n, w = 3000, 4
    js = n // 3
    copies = (js + 17, n // 2 + 5, n - 2)      # n - 2 lies in the window (w = 4)
    near = (js - 40, 2 * n // 3)
    q, k, v = _peaked_with_copies(31 + d, 2, 1, d, n, w, pstar, js, copies, near)
    got = _full_check(ctx, q, k, v, 1, n // 4, f"copies of v* p*={pstar} d={d}")
    assert got is not None
    s, want, _, _ = got
    # the copies score far below their neighbours and match one by one
    for j in copies[:2] + near:
        assert abs(s[0, j] - want[0, j]) <= 2e-3 * want[0, j] + H.FLT_MIN, j


def test_value_rows_copying_the_argmax_llama_shape(ctx):
    """The same at the headline head geometry (G = 4, w = 8: 32 rows), a long head
    over several second-pass chunks, copies of v* in three chunks and pooling."""
    n, w, d = 20011, 8, 128
    js = 4100
    q, k, v = _peaked_with_copies(77, 32, 8, d, n, w, 0.999, js, (5, js + 1, 9000, n - 5),
                                  (12000,))
    _full_check(ctx, q, k, v, 7, n // 20, "copies of v*, 32 rows, n=20011")


@pytest.mark.parametrize("d", [64, 128])
def test_value_rows_with_common_offset(ctx, d):
    """Every value row is a shared offset plus a small per-token part
    (V = 4 mu + 0.05 N(0, 1)): ||a - v_j|| is small against ||a|| and ||v_j|| for
    every token at once, so every distance takes the direct sum."""
    Hq, Hkv, n, w = 8, 2, 3000, 4
    rng = np.random.default_rng(90 + d)
    q = rng.standard_normal((Hq, w, d), dtype=np.float32)
    k = rng.standard_normal((Hkv, n, d), dtype=np.float32)
    mu = rng.standard_normal((Hkv, 1, d), dtype=np.float32)
    v = (4.0 * mu + 0.05 * rng.standard_normal((Hkv, n, d))).astype(np.float32)
    q, k, v = wl.bf16_bits(q), wl.bf16_bits(k), wl.bf16_bits(v)
    _full_check(ctx, q, k, v, 5, n // 10, f"common value offset d={d}")


def test_tied_maxima_across_splits(ctx):
    """Three copies of the dominant key (each holding ~30 % of every row's
    mass) in tiles that the first pass gives to different splits, the lowest
    token in the highest-numbered split: the arg-max is the lowest index and the
    scores match the oracle."""
    d, n = 8, 9000
    splits = dropkv.plan_splits(n, 1)
    rng = np.random.default_rng(11)
    q = np.zeros((2, 2, d), np.float32); q[:, :, 0] = 1.0
    k = np.zeros((1, n, d), np.float32); k[0, :, 1:] = rng.standard_normal((n, d - 1))
    L = math.log(0.3 * n / 0.1)
    tiles = [splits - 1, splits + 1, 3 * splits - 8]   # splits (splits-1), 1, splits-8
    for t in tiles:
        k[0, 32 * t + 3, :] = 0.0
        k[0, 32 * t + 3, 0] = L * math.sqrt(d)
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    q, k, v = wl.bf16_bits(q), wl.bf16_bits(k), wl.bf16_bits(v)
    _full_check(ctx, q, k, v, 3, n // 5, "tied maxima across splits")


def test_nonfinite_rejected(ctx):
    q, k, v = _rand(4, 4, 2, 16, 100, 2)
    for which, idx, val in (("k", 333, 0x7F80), ("v", 17, 0x7FC0), ("q", 5, 0xFF80), ("k", 1500, 0xFF80)):
        arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
        arrs[which].reshape(-1)[idx] = val
        st, *_ = H.gpu_path(ctx, arrs["q"], arrs["k"], arrs["v"], 3, 10, compact=False)
        assert st == dropkv.ENONFINITE, (which, idx, st)


def test_score_beyond_float32_is_erange(ctx):
    q, k, v = _rand(6, 1, 1, 8, 64, 2)
    v = wl.bf16_bits(wl.bf16_to_f32(v) * np.float32(1e36))
    with pytest.raises(orc.OracleError) as e:
        orc.score(q, k, v, 1)
    assert e.value.code == orc.ERANGE
    st, *_ = H.gpu_path(ctx, q, k, v, 1, 10, compact=False)
    assert st == dropkv.ERANGE


@pytest.mark.parametrize("which,val", [("q", 0x5780), ("k", 0xD780), ("v", 0x5780), ("v", 0x577F),
                                       ("k", 0x577F), ("q", 0x7F7F)])
def test_input_contract_matches_oracle(ctx, which, val):
    """Reading R-11: an element of magnitude >= 2^48 is ERANGE on both sides; just
    below it the device reaches the oracle's decision (and, when accepted, its
    scores).  The element sits in a tile of the middle of the sequence."""
    q, k, v = _rand(8, 4, 2, 32, 700, 4)
    arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
    idx = 37 if which == "q" else 300 * 32 + 5
    arrs[which].reshape(-1)[idx] = val
    _full_check(ctx, arrs["q"], arrs["k"], arrs["v"], 3, 100, f"contract {which}={hex(val)}")


def test_input_contract_precedence_on_device(ctx):
    q, k, v = _rand(9, 4, 2, 32, 300, 4)
    a = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
    a["v"].reshape(-1)[1000] = 0x7FC0
    a["k"].reshape(-1)[2000] = 0x5780
    st, *_ = H.gpu_path(ctx, a["q"], a["k"], a["v"], 3, 50, compact=False)
    assert st == dropkv.ENONFINITE
    b = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
    b["q"].reshape(-1)[0] = 0x5780   # out of range, and singular rows
    st, *_ = H.gpu_path(ctx, b["q"], b["k"], b["v"], 3, 50, compact=False)
    assert st == dropkv.ERANGE


def test_back_to_back_calls_with_every_workgroup_resident():
    """Small grids put every first-pass, merge and second-pass workgroup of a
    call on the device at once, so a second-pass workgroup polls its head's
    merge count before the head's splits are even done.  Calls one after the
    other -- each on a fresh context (whose scratch may reuse the last one's
    memory) and then on one context across changing shapes -- must each wait
    for their own counts and match the oracle."""
    shapes = [(8, 8, 96, 1499, 8, 7, 300), (8, 8, 96, 1499, 8, 7, 300), (4, 2, 64, 333, 4, 5, 100),
              (8, 8, 96, 1500, 8, 7, 300), (32, 8, 128, 2600, 8, 7, 900)]
    for i, (Hq, Hkv, d, n, w, pool, budget) in enumerate(shapes):
        c = dropkv.Context(0)
        try:
            q, k, v = _rand(500 + i, Hq, Hkv, d, n, w)
            _full_check(c, q, k, v, pool, budget, f"fresh context {i}: Hq={Hq} Hkv={Hkv} d={d} n={n}")
        finally:
            c.close()
    c = dropkv.Context(0)
    try:
        for i, (Hq, Hkv, d, n, w, pool, budget) in enumerate(shapes + shapes[::-1]):
            q, k, v = _rand(600 + i, Hq, Hkv, d, n, w)
            _full_check(c, q, k, v, pool, budget, f"one context, call {i}: Hq={Hq} Hkv={Hkv} d={d} n={n}")
    finally:
        c.close()


def test_bitwise_deterministic(ctx):
    cfg = wl.LLAMA_4K
    inp = wl.make_layer(cfg, cfg.seed)
    a = H.gpu_path(ctx, inp["q"], inp["k"], inp["v"], cfg.pool, cfg.budget)
    b = H.gpu_path(ctx, inp["q"], inp["k"], inp["v"], cfg.pool, cfg.budget)
    np.testing.assert_array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    np.testing.assert_array_equal(a[2], b[2])


def test_host_argument_checks(ctx):
    q, k, v = _rand(7, 4, 2, 16, 64, 2)
    qd, kd, vd = H.to_dev(q), H.to_dev(k), H.to_dev(v)
    sc = torch.empty((2, 64), dtype=torch.float32, device="cuda")
    bad = [
        dict(Hq=3, Hkv=2), dict(w=0), dict(w=65), dict(pool=2), dict(pool=0), dict(pool=131),
        dict(d=12), dict(d=264), dict(n=0), dict(Hq=130, Hkv=2, w=2),   # G*w = 130 > 128
        dict(Hq=98, Hkv=2, w=2, d=256),                                 # 98 rows at d = 256
    ]
    for b in bad:
        args = dict(n=64, w=2, Hq=4, Hkv=2, d=16, pool=3)
        args.update(b)
        with pytest.raises(dropkv.DropKVError) as e:
            ctx.score(qd, kd, vd, args["n"], args["w"], args["Hq"], args["Hkv"], args["d"],
                      args["pool"], sc)
        assert e.value.code == dropkv.EINVAL, b
    with pytest.raises(dropkv.DropKVError):
        ctx.score(qd.data_ptr() + 2, kd, vd, 64, 2, 4, 2, 16, 3, sc)   # misaligned
    keep = torch.empty((2, 8), dtype=torch.int32, device="cuda")
    for budget in (-1, 65):
        with pytest.raises(dropkv.DropKVError):
            ctx.select(sc, 2, 64, budget, keep)
    assert ctx.sync() == dropkv.OK
