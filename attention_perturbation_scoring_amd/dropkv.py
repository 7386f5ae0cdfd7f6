"""Thin ctypes binding of libdropkv (C ABI in include/dropkv.h).

Argument marshalling only: every step of scoring, selection and compaction runs
in the library's HIP kernels.  Tensors are torch tensors in device memory
(bf16 data may be passed as torch.bfloat16, torch.int16 or torch.uint16 --
only the bit patterns matter); the stream is torch's current stream unless one
is given.  A missing library raises immediately: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdropkv.so")

OK, EINVAL, ESINGULAR, ENONFINITE, ERANGE, EDEVICE, ENOMEM, ESCRATCH = range(8)
KERNELS = ("pass1", "merge", "pass2", "select", "compact", "compact_inplace", "attn_pass1",
           "attn_pass2", "stream_read")


class DropKVError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} (status {code})")


_lib = None


def lib():
    """Load libdropkv.so (built by attention_perturbation_scoring_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libdropkv.so is not built ({LIB_PATH}); run "
                               "`python -m attention_perturbation_scoring_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "dropkv_create": [ctypes.POINTER(P), ctypes.c_int],
            "dropkv_destroy": [P],
            "dropkv_score": [P, P, P, P, i64, i32, i32, i32, i32, i32, P, P],
            "dropkv_score_attention": [P, P, P, i64, i32, i32, i32, i32, i32, P, P],
            "dropkv_score_ex": [P, P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P],
            "dropkv_score_noalloc": [P, P, P, P, i64, i32, i32, i32, i32, i32, P, P],
            "dropkv_select": [P, P, i32, i64, i64, P, P],
            "dropkv_score_select": [P, P, P, P, i64, i32, i32, i32, i32, i32, i64, P, P, P],
            "dropkv_select_layer": [P, P, i32, i64, i64, P, P, P],
            "dropkv_compact": [P, P, P, i32, i64, i32, P, i64, P, P, P],
            "dropkv_compact_inplace": [P, P, P, i32, i64, i64, i32, P, i64, P],
            "dropkv_rescore": [P, P, P, P, i64, i64, i32, i32, i32, i32, i32, i64, P, P, P],
            "dropkv_sync": [P, P],
            "dropkv_set_select_wait": [P, i64],
            "dropkv_profile_enable": [P, ctypes.c_int],
            "dropkv_profile_reset": [P],
            "dropkv_profile_read": [P, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)],
            "dropkv_plan_splits": [i64, i32, ctypes.POINTER(i32)],
            "dropkv_scratch_bytes": [i64, i32, i32, i32, i32, ctypes.POINTER(i64),
                                     ctypes.POINTER(i64)],
            "dropkv_stream_read": [P, P, i64, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.dropkv_noalloc_scratch_bytes.argtypes = []
        L.dropkv_noalloc_scratch_bytes.restype = ctypes.c_int64
        L.dropkv_strerror.argtypes = [ctypes.c_int]
        L.dropkv_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    try:
        return lib().dropkv_strerror(code).decode()
    except RuntimeError:
        return f"status {code}"


def _check(rc: int, what: str):
    if rc != OK:
        raise DropKVError(rc, what)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("tensor must be in device memory")
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def plan_splits(n: int, Hkv: int) -> int:
    s = ctypes.c_int32(0)
    _check(lib().dropkv_plan_splits(n, Hkv, ctypes.byref(s)), "dropkv_plan_splits")
    return s.value


def scratch_bytes(n: int, w: int, Hq: int, Hkv: int, d: int):
    """(score scratch, select scratch) in bytes that a context holds for these sizes."""
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().dropkv_scratch_bytes(n, w, Hq, Hkv, d, ctypes.byref(a), ctypes.byref(b)),
           "dropkv_scratch_bytes")
    return a.value, b.value


class Context:
    """Owns a dropkv_ctx (scratch + device error latch) on one device."""

    def __init__(self, device: int | None = None):
        if device is None:
            device = torch.cuda.current_device()
        self.device = device
        h = ctypes.c_void_p()
        _check(lib().dropkv_create(ctypes.byref(h), device), "dropkv_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().dropkv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- the three calls of the path --
    def score(self, q_win, k_cache, v_cache, n, w, Hq, Hkv, d, pool, scores, stream=None):
        _check(lib().dropkv_score(self._h, _ptr(q_win), _ptr(k_cache), _ptr(v_cache), n, w, Hq,
                                  Hkv, d, pool, _ptr(scores), _stream(stream)), "dropkv_score")

    def score_noalloc(self, q_win, k_cache, v_cache, n, w, Hq, Hkv, d, pool, scores, stream=None):
        _check(lib().dropkv_score_noalloc(self._h, _ptr(q_win), _ptr(k_cache), _ptr(v_cache), n, w,
                                          Hq, Hkv, d, pool, _ptr(scores), _stream(stream)),
               "dropkv_score_noalloc")

    def score_ex(self, q_win, k_cache, v_cache, n, w, Hq, Hkv, d, pool, scores, out_a=None,
                 out_lse=None, stream=None):
        _check(lib().dropkv_score_ex(self._h, _ptr(q_win), _ptr(k_cache), _ptr(v_cache), n, w, Hq,
                                     Hkv, d, pool, _ptr(scores), _ptr(out_a), _ptr(out_lse),
                                     _stream(stream)), "dropkv_score_ex")

    def score_attention(self, q_win, k_cache, n, w, Hq, Hkv, d, pool, scores, stream=None):
        _check(lib().dropkv_score_attention(self._h, _ptr(q_win), _ptr(k_cache), n, w, Hq, Hkv, d,
                                            pool, _ptr(scores), _stream(stream)),
               "dropkv_score_attention")

    def score_select(self, q_win, k_cache, v_cache, n, w, Hq, Hkv, d, pool, budget, scores, keep,
                     stream=None):
        _check(lib().dropkv_score_select(self._h, _ptr(q_win), _ptr(k_cache), _ptr(v_cache), n, w,
                                         Hq, Hkv, d, pool, budget, _ptr(scores), _ptr(keep),
                                         _stream(stream)), "dropkv_score_select")

    def select(self, scores, Hkv, n, budget, keep, stream=None):
        _check(lib().dropkv_select(self._h, _ptr(scores), Hkv, n, budget, _ptr(keep),
                                   _stream(stream)), "dropkv_select")

    def select_layer(self, scores, Hkv, n, budget, keep, counts, stream=None):
        _check(lib().dropkv_select_layer(self._h, _ptr(scores), Hkv, n, budget, _ptr(keep),
                                         _ptr(counts), _stream(stream)), "dropkv_select_layer")

    def compact(self, k, v, Hkv, n, d, keep, budget, k_out, v_out, stream=None):
        _check(lib().dropkv_compact(self._h, _ptr(k), _ptr(v), Hkv, n, d, _ptr(keep), budget,
                                    _ptr(k_out), _ptr(v_out), _stream(stream)), "dropkv_compact")

    def compact_inplace(self, k_cache, v_cache, Hkv, cap, n_valid, d, keep, budget, stream=None):
        _check(lib().dropkv_compact_inplace(self._h, _ptr(k_cache), _ptr(v_cache), Hkv, cap, n_valid,
                                            d, _ptr(keep), budget, _stream(stream)),
               "dropkv_compact_inplace")

    def rescore(self, q_win, k_cache, v_cache, cap, n_valid, w, Hq, Hkv, d, pool, budget, scores,
                keep, stream=None):
        _check(lib().dropkv_rescore(self._h, _ptr(q_win), _ptr(k_cache), _ptr(v_cache), cap, n_valid,
                                    w, Hq, Hkv, d, pool, budget, _ptr(scores), _ptr(keep),
                                    _stream(stream)), "dropkv_rescore")

    def stream_read(self, buf, nbytes=None, stream=None):
        """Read a device buffer once (the achievable-bandwidth reference)."""
        nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
        _check(lib().dropkv_stream_read(self._h, _ptr(buf), nbytes, _stream(stream)),
               "dropkv_stream_read")

    def set_select_wait(self, polls: int):
        """Team-barrier polls before a selection workgroup finishes its share alone."""
        _check(lib().dropkv_set_select_wait(self._h, polls), "dropkv_set_select_wait")

    def sync(self, stream=None) -> int:
        """Wait for the stream; return (and clear) the latched device status."""
        return lib().dropkv_sync(self._h, _stream(stream))

    def check(self, stream=None):
        _check(self.sync(stream), "device")

    # -- measurement hooks --
    def profile(self, on: bool = True):
        _check(lib().dropkv_profile_enable(self._h, 1 if on else 0), "dropkv_profile_enable")

    def profile_reset(self):
        _check(lib().dropkv_profile_reset(self._h), "dropkv_profile_reset")

    def profile_read(self, name: str):
        ms, cnt = ctypes.c_double(0.0), ctypes.c_int64(0)
        _check(lib().dropkv_profile_read(self._h, name.encode(), ctypes.byref(ms), ctypes.byref(cnt)),
               "dropkv_profile_read")
        return ms.value, cnt.value


# Module-level aliases with the C names.
def dropkv_score(ctx: Context, *args, **kw):
    return ctx.score(*args, **kw)


def dropkv_score_ex(ctx: Context, *args, **kw):
    return ctx.score_ex(*args, **kw)


def dropkv_score_attention(ctx: Context, *args, **kw):
    return ctx.score_attention(*args, **kw)


def dropkv_select(ctx: Context, *args, **kw):
    return ctx.select(*args, **kw)


def dropkv_score_select(ctx: Context, *args, **kw):
    return ctx.score_select(*args, **kw)


def dropkv_select_layer(ctx: Context, *args, **kw):
    return ctx.select_layer(*args, **kw)


def dropkv_compact(ctx: Context, *args, **kw):
    return ctx.compact(*args, **kw)


def dropkv_compact_inplace(ctx: Context, *args, **kw):
    return ctx.compact_inplace(*args, **kw)


def dropkv_rescore(ctx: Context, *args, **kw):
    return ctx.rescore(*args, **kw)


def dropkv_stream_read(ctx: Context, *args, **kw):
    return ctx.stream_read(*args, **kw)


def dropkv_sync(ctx: Context, stream=None) -> int:
    return ctx.sync(stream)


def run_path(ctx: Context, q, k, v, n, w, Hq, Hkv, d, pool, budget, stream=None):
    """score -> select -> compact on device tensors; returns (scores, keep, k_out, v_out).

    Allocates the outputs with torch; raises on a latched device condition.
    """
    dev = k.device
    scores = torch.empty((Hkv, n), dtype=torch.float32, device=dev)
    keep = torch.empty((Hkv, budget), dtype=torch.int32, device=dev)
    k_out = torch.empty((Hkv, budget, d), dtype=k.dtype, device=dev)
    v_out = torch.empty((Hkv, budget, d), dtype=v.dtype, device=dev)
    ctx.score(q, k, v, n, w, Hq, Hkv, d, pool, scores, stream)
    ctx.select(scores, Hkv, n, budget, keep, stream)
    ctx.compact(k, v, Hkv, n, d, keep, budget, k_out, v_out, stream)
    ctx.check(stream)
    return scores, keep, k_out, v_out
