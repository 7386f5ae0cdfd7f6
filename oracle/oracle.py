"""ctypes front end of the float64 CPU oracle (oracle/dropkv_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  It shares no code
with the HIP path.

All functions take numpy arrays of bf16 bit patterns (uint16) in the layouts
q [Hq][w][d], k/v [Hkv][n][d] and return float64 / int32 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dropkv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

OK, EINVAL, ESINGULAR, ENONFINITE, ERANGE, ENOMEM = 0, 1, 2, 3, 4, 6
NAMES = {OK: "OK", EINVAL: "EINVAL", ESINGULAR: "ESINGULAR", ENONFINITE: "ENONFINITE",
         ERANGE: "ERANGE", ENOMEM: "ENOMEM"}


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle returned {NAMES.get(code, code)}")
        self.code = code


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over KV heads)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def load(path: str):
    """Open an oracle shared object and declare its signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    L.oracle_raw_scores.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P]
    L.oracle_pool_protect.argtypes = [P, i64, i32, i32, i32, P]
    L.oracle_score.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, i32, P]
    L.oracle_select.argtypes = [P, i32, i64, i64, P]
    L.oracle_compact.argtypes = [P, i32, i64, i32, P, i64, P]
    L.oracle_window_attention.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P]
    L.oracle_attention_raw.argtypes = [P, P, i64, i32, i32, i32, i32, i32, P]
    L.oracle_window_lse.argtypes = [P, P, i64, i32, i32, i32, i32, P]
    L.oracle_select_layer.argtypes = [P, i32, i64, i64, P, P]
    L.oracle_attention_score.argtypes = [P, P, i64, i32, i32, i32, i32, i32, i32, P]
    L.oracle_compact_inplace.argtypes = [P, i32, i64, i64, i32, P, i64]
    L.oracle_rescore.argtypes = [P, P, P, i64, i64, i32, i32, i32, i32, i32, i32, P]
    for f in (L.oracle_raw_scores, L.oracle_pool_protect, L.oracle_score, L.oracle_select,
              L.oracle_compact, L.oracle_window_attention, L.oracle_compact_inplace,
              L.oracle_rescore):
        f.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        _lib = load(LIB)
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def _check(rc):
    if rc != OK:
        raise OracleError(rc)


def _dims(q, k):
    Hq, w, d = q.shape
    Hkv, n, d2 = k.shape
    assert d == d2
    return Hq, w, d, Hkv, n


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def raw_scores(q, k, v, nthreads=None):
    """Head-averaged, window-summed ||Delta_j||^2 before pooling: float64 [Hkv][n]."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    Hq, w, d, Hkv, n = _dims(q, k)
    out = np.zeros((Hkv, n), dtype=np.float64)
    _check(lib().oracle_raw_scores(_ptr(q), _ptr(k), _ptr(v), n, w, Hq, Hkv, d,
                                   nthreads or default_threads(), _ptr(out)))
    return out


def pool_protect(raw, w, pool):
    raw = np.ascontiguousarray(raw, dtype=np.float64)
    Hkv, n = raw.shape
    out = np.zeros_like(raw)
    _check(lib().oracle_pool_protect(_ptr(raw), n, Hkv, w, pool, _ptr(out)))
    return out


def score(q, k, v, pool, nthreads=None):
    """Final scores (pooled, window = +inf): float64 [Hkv][n]."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    Hq, w, d, Hkv, n = _dims(q, k)
    out = np.zeros((Hkv, n), dtype=np.float64)
    _check(lib().oracle_score(_ptr(q), _ptr(k), _ptr(v), n, w, Hq, Hkv, d, pool,
                              nthreads or default_threads(), _ptr(out)))
    return out


def attention_raw(q, k, nthreads=None):
    """Attention-only raw scores: head-averaged, window-summed p_j. float64 [Hkv][n]."""
    q, k = _u16(q), _u16(k)
    Hq, w, d, Hkv, n = _dims(q, k)
    out = np.zeros((Hkv, n), dtype=np.float64)
    _check(lib().oracle_attention_raw(_ptr(q), _ptr(k), n, w, Hq, Hkv, d,
                                      nthreads or default_threads(), _ptr(out)))
    return out


def attention_score(q, k, pool, nthreads=None):
    """Attention-only final scores (pooled, window = +inf): float64 [Hkv][n]."""
    q, k = _u16(q), _u16(k)
    Hq, w, d, Hkv, n = _dims(q, k)
    out = np.zeros((Hkv, n), dtype=np.float64)
    _check(lib().oracle_attention_score(_ptr(q), _ptr(k), n, w, Hq, Hkv, d, pool,
                                        nthreads or default_threads(), _ptr(out)))
    return out


def select(scores, budget):
    """Kept indices per head, ascending: int32 [Hkv][budget]."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    Hkv, n = s.shape
    keep = np.zeros((Hkv, budget), dtype=np.int32)
    _check(lib().oracle_select(_ptr(s), Hkv, n, budget, _ptr(keep)))
    return keep


def select_layer(scores, budget):
    """Layer-wide selection: (flat kept indices g*n + j ascending int32 [budget],
    per-head counts int32 [Hkv])."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    Hkv, n = s.shape
    keep = np.zeros(max(budget, 1), dtype=np.int32)
    counts = np.zeros(Hkv, dtype=np.int32)
    _check(lib().oracle_select_layer(_ptr(s), Hkv, n, budget, _ptr(keep), _ptr(counts)))
    return keep[:budget], counts


def compact(x, keep):
    x = _u16(x)
    keep = np.ascontiguousarray(keep, dtype=np.int32)
    Hkv, n, d = x.shape
    budget = keep.shape[1]
    out = np.zeros((Hkv, budget, d), dtype=np.uint16)
    _check(lib().oracle_compact(_ptr(x), Hkv, n, d, _ptr(keep), budget, _ptr(out)))
    return out


def compact_inplace(cache, keep, n_valid):
    """In-place compaction of a resident cache [Hkv][cap][d] (uint16, modified
    in place and returned): row r of head g becomes old row keep[g][r]."""
    assert cache.dtype == np.uint16 and cache.flags.c_contiguous
    keep = np.ascontiguousarray(keep, dtype=np.int32)
    Hkv, cap, d = cache.shape
    budget = keep.shape[1]
    _check(lib().oracle_compact_inplace(_ptr(cache), Hkv, cap, n_valid, d, _ptr(keep), budget))
    return cache


def rescore(q, k, v, n_valid, pool, nthreads=None):
    """Scores [Hkv][n_valid] (float64) of the first n_valid rows of resident
    caches k, v [Hkv][cap][d]; the window is the last w of those rows."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    Hq, w, d = q.shape
    Hkv, cap, _ = k.shape
    out = np.zeros((Hkv, n_valid), dtype=np.float64)
    _check(lib().oracle_rescore(_ptr(q), _ptr(k), _ptr(v), cap, n_valid, w, Hq, Hkv, d, pool,
                                nthreads or default_threads(), _ptr(out)))
    return out


def window_attention(q, k, v):
    """(p [Hq][w][n], a [Hq][w][d], s_excl [Hq][w]) in float64."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    Hq, w, d, Hkv, n = _dims(q, k)
    p = np.zeros((Hq, w, n))
    a = np.zeros((Hq, w, d))
    sx = np.zeros((Hq, w))
    _check(lib().oracle_window_attention(_ptr(q), _ptr(k), _ptr(v), n, w, Hq, Hkv, d,
                                         _ptr(p), _ptr(a), _ptr(sx)))
    return p, a, sx


def window_lse(q, k):
    """Natural-log log-sum-exp of each window query's visible logits: float64 [Hq][w]."""
    q, k = _u16(q), _u16(k)
    Hq, w, d, Hkv, n = _dims(q, k)
    out = np.zeros((Hq, w))
    _check(lib().oracle_window_lse(_ptr(q), _ptr(k), n, w, Hq, Hkv, d, _ptr(out)))
    return out


def max_probability(q, k, v) -> float:
    """Largest attention probability over all window queries and visible keys."""
    p, _, _ = window_attention(q, k, v)
    return float(p.max())
