"""The C ABI library loads and exports every entry point include/dropkv.h
declares; host-only entry points behave without a GPU."""
import os
import re
import subprocess

import pytest

from attention_perturbation_scoring_amd import dropkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dropkv.h")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char \*)\s*(dropkv_\w+)\s*\(", text,
                                 re.M)))


def test_header_declares_the_path():
    names = declared()
    for must in ("dropkv_create", "dropkv_destroy", "dropkv_score", "dropkv_select",
                 "dropkv_compact", "dropkv_sync", "dropkv_strerror"):
        assert must in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(dropkv.LIB_PATH):
        pytest.skip("libdropkv.so not built")
    out = subprocess.run(["nm", "-D", "--defined-only", dropkv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(dropkv_\w+)$", out, re.M))
    missing = [n for n in declared() if n not in exported]
    assert not missing, missing
    L = dropkv.lib()
    for n in declared():
        assert hasattr(L, n)


def test_host_only_entry_points():
    if not os.path.exists(dropkv.LIB_PATH):
        pytest.skip("libdropkv.so not built")
    assert dropkv.strerror(dropkv.ESINGULAR).startswith("a window query")
    assert dropkv.strerror(12345) == "unknown status"
    assert dropkv.plan_splits(131072, 8) == 64
    assert dropkv.plan_splits(22, 2) == 1
    assert dropkv.plan_splits(4096, 8) == 16
    L = dropkv.lib()
    assert L.dropkv_score(None, None, None, None, 10, 1, 1, 1, 8, 1, None, None) == dropkv.EINVAL
    assert L.dropkv_sync(None, None) == dropkv.EINVAL
    assert L.dropkv_stream_read(None, None, 16, None) == dropkv.EINVAL
    assert L.dropkv_score_noalloc(None, None, None, None, 10, 1, 1, 1, 8, 1, None, None) == dropkv.EINVAL
    assert L.dropkv_noalloc_scratch_bytes() == 16 << 20
    # in-place compaction and rescoring reject a missing context on the host
    assert L.dropkv_compact_inplace(None, None, None, 1, 10, 10, 8, None, 5, None) == dropkv.EINVAL
    assert L.dropkv_rescore(None, None, None, None, 10, 10, 1, 1, 1, 8, 1, 5, None, None,
                            None) == dropkv.EINVAL
    assert L.dropkv_score_select(None, None, None, None, 10, 1, 1, 1, 8, 1, 5, None, None,
                                 None) == dropkv.EINVAL
    assert dropkv.strerror(dropkv.ESCRATCH).startswith("needs more scratch")
    # scratch at the headline shape: 64 splits x 32 rows x (d + 5) floats per KV
    # head, per-row state and the merge helpers' parts -- megabytes (within the
    # no-allocation entry point's static buffer), nothing of size n * d
    sb, selb = dropkv.scratch_bytes(131072, 8, 32, 8, 128)
    assert 8 * 64 * 32 * (128 + 5) * 4 <= sb <= L.dropkv_noalloc_scratch_bytes()
    assert 0 < selb < 4 * 2**20
    with pytest.raises(dropkv.DropKVError):
        dropkv.scratch_bytes(100, 8, 3, 2, 128)     # Hq % Hkv != 0


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    monkeypatch.setattr(dropkv, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(dropkv, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        dropkv.lib()
