"""Seeded synthetic workloads for DropKV scoring (inputs only, no scoring arithmetic).

This module is the one place that draws inputs. Both the HIP path and the fp64
CPU oracle consume the exact bytes it produces, so it deliberately holds none of
the method's arithmetic: no softmax, no perturbation, no pooling, no selection.

Shapes follow the paper's evaluation setup (DropKV, arXiv 2610.22130: Section 5
"Experiments" uses B=1, an observation window of w=8 tail queries and 5/10 %
budgets; Section 5.4 and Figure 3 time the scoring step at n = 4K ... 128K on
Llama-3.1-8B-shaped heads).  Real model activations are not available, so the
values are synthetic:

* Q, K, V are i.i.d. standard normal float32 draws from numpy's PCG64,
  drawn in the order Q [Hq][w][d], K [Hkv][n][d], V [Hkv][n][d].
* "outlier" workloads then scale 4 channels of K by 8 in every KV head
  (channels drawn per head with ``rng.choice(d, 4, replace=False)``).  Only K is
  scaled: scaling the same channels of Q as well makes nearly every row's
  softmax collapse onto one token, which is not what long-context attention
  looks like.
* "sink" workloads then add to keys 0..3 of every KV head the least-norm vector
  b_g that raises every window query's logit by +6 (q . b_g / sqrt(d) = 6 for all
  G*w queries of the group, solved in float64 with ``numpy.linalg.lstsq``).
* "sink-heavy" workloads (recipe ``llama_sink``) do all of the above and then
  replace key 0 of every KV head by the least-norm vector that sets every
  window query's logit on it to 20 (float64 least squares): at 128K tokens
  every window query then puts p > 0.99 on token 0, an attention-sink pattern
  strong enough that each row's arg-max holds more than 0.94 of its mass.
* Everything is finally rounded to bfloat16 (round to nearest, ties to even).
  Both sides see only these bf16 bytes.

Layouts: q_win is [L*Hq][w][d], k and v are [L*Hkv][n][d], all uint16 holding
bf16 bit patterns.  Layers (L) fold into heads.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Callable, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    Hq: int
    Hkv: int
    d: int
    n: int
    w: int
    pool: int
    budget: int          # kept tokens per KV head (includes the protected window)
    seed: int
    layers: int = 1
    recipe: str = "llama"  # "tiny" (plain normal + acceptance predicate), "llama" or "llama_sink"

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def heads_kv(self) -> int:
        return self.layers * self.Hkv

    @property
    def heads_q(self) -> int:
        return self.layers * self.Hq

    @property
    def evict(self) -> int:
        return self.n - self.budget


def budget_for(n: int, pct: float) -> int:
    """Kept tokens per head: floor(pct * n / 100), the window included."""
    return int(np.floor(pct * n / 100.0))


# The five workloads: a tiny case for exhaustive checks, and Llama-3.1-8B /
# Phi-3-mini shaped single-layer and full-cache cases.
TINY = Config("tiny", Hq=4, Hkv=2, d=8, n=22, w=3, pool=3, budget=15, seed=42, recipe="tiny")
LLAMA_4K = Config("llama4k", Hq=32, Hkv=8, d=128, n=4096, w=8, pool=7,
                  budget=budget_for(4096, 5), seed=7)
LLAMA_32K = Config("llama32k", Hq=32, Hkv=8, d=128, n=32768, w=8, pool=7,
                   budget=budget_for(32768, 10), seed=8)
LLAMA_128K = Config("llama128k", Hq=32, Hkv=8, d=128, n=131072, w=8, pool=7,
                    budget=budget_for(131072, 5), seed=9)
PHI3_FULL = Config("phi3full", Hq=32, Hkv=32, d=96, n=131072, w=8, pool=7,
                   budget=budget_for(131072, 5), seed=1000, layers=32)
# Sink-heavy variants of the Llama cases: every window row's arg-max (token 0)
# holds more than 0.94 of its attention.
LLAMA_4K_SINK = Config("llama4k_sink", Hq=32, Hkv=8, d=128, n=4096, w=8, pool=7,
                       budget=budget_for(4096, 5), seed=17, recipe="llama_sink")
LLAMA_128K_SINK = Config("llama128k_sink", Hq=32, Hkv=8, d=128, n=131072, w=8, pool=7,
                         budget=budget_for(131072, 5), seed=19, recipe="llama_sink")

CONFIGS = {c.name: c for c in (TINY, LLAMA_4K, LLAMA_32K, LLAMA_128K, PHI3_FULL, LLAMA_4K_SINK,
                               LLAMA_128K_SINK)}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN stays NaN (quiet), +-inf stays +-inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    # NaN bit patterns near 0xFFFFFFFF would wrap in uint32; they are fixed below
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _outliers_and_sinks(rng, q32, k32, Hkv, G, w, d, n_sinks=4, boost=6.0, scale=8.0):
    """In place on float32 arrays of one layer: K outlier channels, then sink keys."""
    for g in range(Hkv):
        ch = rng.choice(d, 4, replace=False)
        k32[g][:, ch] *= np.float32(scale)
    n_s = min(n_sinks, k32.shape[1])
    for g in range(Hkv):
        qg = q32[g * G:(g + 1) * G].reshape(G * w, d).astype(np.float64)
        rhs = np.full(G * w, boost * np.sqrt(d), dtype=np.float64)
        b, *_ = np.linalg.lstsq(qg, rhs, rcond=None)
        k32[g][:n_s] += b.astype(np.float32)[None, :]


def _heavy_sink(q32, k32, Hkv, G, w, d, logit=20.0):
    """In place: key 0 of every KV head becomes the least-norm vector that sets
    every window query's logit on it to `logit` (float64 least squares)."""
    for g in range(Hkv):
        qg = q32[g * G:(g + 1) * G].reshape(G * w, d).astype(np.float64)
        rhs = np.full(G * w, logit * np.sqrt(d), dtype=np.float64)
        b, *_ = np.linalg.lstsq(qg, rhs, rcond=None)
        k32[g][0] = b.astype(np.float32)


def make_layer(cfg: Config, seed: int, accept: Optional[Callable] = None, max_tries: int = 1000):
    """One layer's bf16 inputs: dict(q=[Hq][w][d], k=[Hkv][n][d], v=[Hkv][n][d], tries=int).

    For the "tiny" recipe, ``accept(q, k, v) -> bool`` (if given) decides whether a
    draw is kept; rejected draws are replaced by the next draws from the same
    generator stream.  The predicate is supplied by the caller (for the paper's
    tiny case: no probability above 0.5), so this module computes none of it.
    """
    rng = np.random.default_rng(seed)
    for tries in range(1, max_tries + 1):
        q32 = _draw_normal(rng, (cfg.Hq, cfg.w, cfg.d))
        k32 = _draw_normal(rng, (cfg.Hkv, cfg.n, cfg.d))
        v32 = _draw_normal(rng, (cfg.Hkv, cfg.n, cfg.d))
        if cfg.recipe in ("llama", "llama_sink"):
            _outliers_and_sinks(rng, q32, k32, cfg.Hkv, cfg.G, cfg.w, cfg.d)
        if cfg.recipe == "llama_sink":
            _heavy_sink(q32, k32, cfg.Hkv, cfg.G, cfg.w, cfg.d)
        q, k, v = bf16_bits(q32), bf16_bits(k32), bf16_bits(v32)
        del q32, k32, v32
        if accept is None or accept(q, k, v):
            return dict(q=q, k=k, v=v, tries=tries)
    raise RuntimeError(f"no accepted draw in {max_tries} tries for {cfg.name}")


def layer_seed(cfg: Config, layer: int) -> int:
    return cfg.seed + layer if cfg.layers > 1 else cfg.seed


def make_inputs(cfg: Config, accept: Optional[Callable] = None):
    """All layers, folded into heads: q [L*Hq][w][d], k, v [L*Hkv][n][d] (uint16)."""
    if cfg.layers == 1:
        return make_layer(cfg, cfg.seed, accept)
    parts = [make_layer(cfg, layer_seed(cfg, i), accept) for i in range(cfg.layers)]
    return dict(q=np.concatenate([p["q"] for p in parts]),
                k=np.concatenate([p["k"] for p in parts]),
                v=np.concatenate([p["v"] for p in parts]),
                tries=max(p["tries"] for p in parts))


def digest(arrs) -> str:
    h = hashlib.sha256()
    for a in arrs:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def custom(Hq, Hkv, d, n, w, pool, budget, seed, recipe="tiny", layers=1) -> Config:
    return Config(f"custom_{Hq}_{Hkv}_{d}_{n}_{w}", Hq=Hq, Hkv=Hkv, d=d, n=n, w=w, pool=pool,
                  budget=budget, seed=seed, layers=layers, recipe=recipe)
