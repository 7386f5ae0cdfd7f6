"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the float64 oracle on the same bf16 bytes."""
from __future__ import annotations

import numpy as np
import torch

from attention_perturbation_scoring_amd import dropkv

RTOL = 2e-3                         # fp32 accumulation vs float64 (relative, per score)
FLT_MIN = float(np.finfo(np.float32).tiny)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


GUARD = 256   # sentinel elements on each side of every output buffer
_BITS = {torch.float32: torch.int32, torch.int32: torch.int32, torch.int16: torch.int16}
_SENTINEL = {torch.int32: 0x7FBEEF01, torch.int16: 0x5A5B}   # a NaN pattern for fp32 outputs


class Guarded:
    """An output tensor inside one allocation with GUARD sentinel elements
    before and after it: a kernel that writes past either end of its output
    changes a sentinel, which check() reports."""

    def __init__(self, shape, dtype, fill=0):
        shape = tuple(int(x) for x in shape)
        self.numel = int(np.prod(shape)) if shape else 1
        self.buf = torch.empty(self.numel + 2 * GUARD, dtype=dtype, device="cuda")
        self.bits = _BITS[dtype]
        self.buf.view(self.bits).fill_(_SENTINEL[self.bits])
        self.t = self.buf[GUARD:GUARD + self.numel].view(shape)
        self.t.fill_(fill)

    def check(self, what=""):
        b = self.buf.view(self.bits)
        head, tail = b[:GUARD], b[GUARD + self.numel:]
        sent = _SENTINEL[self.bits]
        assert bool((head == sent).all()), f"{what}: write before the start of the output"
        assert bool((tail == sent).all()), f"{what}: write past the end of the output"


def gpu_path(ctx, q, k, v, pool, budget, select=True, compact=True):
    """Returns (status, scores fp32 [Hkv][n], keep int32 [Hkv][budget] or None,
    k_out, v_out uint16 or None) computed by libdropkv."""
    Hq, w, d = q.shape
    Hkv, n, _ = k.shape
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    outs = dict(scores=Guarded((Hkv, n), torch.float32, -7.0),
                keep=Guarded((Hkv, max(budget, 1)), torch.int32, -5),
                k_out=Guarded((Hkv, max(budget, 1), d), torch.int16),
                v_out=Guarded((Hkv, max(budget, 1), d), torch.int16))
    scores, keep, ko, vo = (outs[x].t for x in ("scores", "keep", "k_out", "v_out"))
    ctx.score(qd, kd, vd, n, w, Hq, Hkv, d, pool, scores)
    if select:
        ctx.select(scores, Hkv, n, budget, keep)
    if select and compact:
        ctx.compact(kd, vd, Hkv, n, d, keep, budget, ko, vo)
    st = ctx.sync()
    torch.cuda.synchronize()
    for name, g in outs.items():
        g.check(name)
    s = scores.cpu().numpy()
    kp = keep.cpu().numpy()[:, :budget] if select else None
    kk = ko.cpu().numpy().view(np.uint16)[:, :budget] if (select and compact) else None
    vv = vo.cpu().numpy().view(np.uint16)[:, :budget] if (select and compact) else None
    return st, s, kp, kk, vv


def assert_scores_close(got: np.ndarray, want: np.ndarray, rtol=RTOL, where=""):
    """Finite oracle scores: |got - want| <= rtol |want| + FLT_MIN; +inf must match."""
    inf = np.isinf(want)
    assert np.array_equal(np.isinf(got), inf), f"{where}: +inf positions differ"
    assert np.all(got[inf] > 0), f"{where}: -inf where +inf expected"
    g, w_ = got[~inf].astype(np.float64), want[~inf]
    err = np.abs(g - w_)
    bound = rtol * np.abs(w_) + FLT_MIN
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err / bound))
        raise AssertionError(f"{where}: {int(bad.sum())} scores outside tolerance; worst "
                             f"got={g[i]!r} want={w_[i]!r} rel={err[i] / max(abs(w_[i]), 1e-300):.3e}")


def assert_keep_sets_match(keep_gpu, keep_orc, scores_orc, budget, rtol=RTOL, where=""):
    """Evicted sets equal except for tokens whose oracle score is within rtol of
    the oracle's k-th smallest score (the decision boundary)."""
    Hkv, n = scores_orc.shape
    k_ev = n - budget
    for g in range(Hkv):
        kg = np.sort(keep_gpu[g])
        assert len(np.unique(kg)) == budget, f"{where}: head {g} keep has duplicates"
        assert np.all((kg >= 0) & (kg < n)), f"{where}: head {g} keep out of range"
        assert np.all(np.diff(keep_gpu[g]) > 0), f"{where}: head {g} keep not ascending"
        if k_ev == 0:
            continue
        s = scores_orc[g]
        T = np.partition(s, k_ev - 1)[k_ev - 1]   # the k-th smallest score
        band = np.abs(s - T) <= rtol * abs(T)
        ev_g = np.ones(n, bool); ev_g[kg] = False
        ev_o = np.ones(n, bool); ev_o[keep_orc[g]] = False
        diff = (ev_g != ev_o) & ~band
        assert not diff.any(), f"{where}: head {g}: {int(diff.sum())} eviction decisions differ outside the band"


def ctx():
    return dropkv.Context(0)
