"""The oracle's pins are sensitive: plant one plausible mistake at a time in a
copy of the oracle source (built here on the CPU, never used anywhere else) and
check that at least one pin then fails.  The shipped oracle is untouched."""
import os
import subprocess

import numpy as np
import pytest
import torch

from attention_perturbation_scoring_amd import workload as wl
from oracle import oracle as orc
import brute

MUTANTS = {
    # name: (exact text in the oracle, replacement)
    "odds_not_squared": ("c = odds * odds * dist2;", "c = odds * dist2;"),
    "one_minus_p_sign": ("(S - l[j]) / S;", "(S + l[j]) / S;"),
    "causal_off_by_one": ("const int64_t P = n - w + t; /* last key", "const int64_t P = n - w + t - 1; /* last key"),
    "no_head_mean": ("rg[j] /= (double)G;", "rg[j] /= 1.0;"),
    "strided_head_groups": ("const int h = g * G + row / w, t = row % w;",
                            "const int h = g + (row / w) * hkv, t = row % w;"),
    "argmax_form_unsquared_p": ("c = pj * pj * dist2;", "c = pj * dist2;"),
    "residual_sign_abar": ("const double r = abar[i] - V[j * d + i];", "const double r = abar[i] + V[j * d + i];"),
    "no_sqrt_d": ("l[j] = s * inv_sqrt_d;\n    }\n    /* maximum", "l[j] = s;\n    }\n    /* maximum"),
    "pool_radius": ("const int64_t r = (pool - 1) / 2;", "const int64_t r = (pool + 1) / 2;"),
    "protect_one_short": ("y[j] = (j >= n - w) ? INFINITY : mx;", "y[j] = (j > n - w) ? INFINITY : mx;"),
    "ties_newest_first": ("return (a->j > b->j) - (a->j < b->j);", "return (a->j < b->j) - (a->j > b->j);"),
    # attention-only scores
    "attn_no_head_mean": ("rg[j] = rg[j] / (double)G;", "rg[j] = rg[j];"),
    "attn_causal_off_by_one": ("const int64_t Pt = n - w + t;", "const int64_t Pt = n - w + t - 1;"),
    "attn_no_sqrt_d": ("l[j] = inv_sqrt_d * s;", "l[j] = s;"),
    "attn_unnormalised": ("rg[j] += l[j] / S;", "rg[j] += l[j];"),
    # decode-time pieces
    "inplace_descending": ("for (int64_t r = 0; r < budget; ++r) {\n            const int64_t j = keep[(size_t)g * budget + r];\n            if (j != r)",
                           "for (int64_t r = budget - 1; r >= 0; --r) {\n            const int64_t j = keep[(size_t)g * budget + r];\n            if (j != r)"),
    "rescore_head_stride": ("memcpy(kr + (size_t)g * n_valid * d, k + (size_t)g * cap * d,",
                            "memcpy(kr + (size_t)g * n_valid * d, k + (size_t)g * n_valid * d,"),
}


def _pins_pass(L):
    """Run a compact set of the pins against library L; True if all hold."""
    saved = orc._lib
    orc._lib = L
    try:
        rng = np.random.default_rng(123)
        q = wl.bf16_bits(rng.standard_normal((4, 3, 8), dtype=np.float32))
        k = wl.bf16_bits(rng.standard_normal((2, 17, 8), dtype=np.float32))
        v = wl.bf16_bits(rng.standard_normal((2, 17, 8), dtype=np.float32))
        if not np.allclose(orc.raw_scores(q, k, v), brute.deletion_raw(q, k, v), rtol=1e-9, atol=0):
            return False
        # a peaked row exercises the arg-max form
        q2 = np.zeros((1, 1, 8), np.float32); q2[0, 0, 0] = 1
        k2 = rng.standard_normal((1, 12, 8)).astype(np.float32); k2[0, :, 0] = 0; k2[0, 0, 0] = 6.0 * np.sqrt(8)
        v2 = rng.standard_normal((1, 12, 8)).astype(np.float32)
        q2, k2, v2 = wl.bf16_bits(q2), wl.bf16_bits(k2), wl.bf16_bits(v2)
        if not np.allclose(orc.raw_scores(q2, k2, v2), brute.deletion_raw(q2, k2, v2), rtol=1e-8, atol=0):
            return False
        raw = rng.random((2, 30)) * (rng.random((2, 30)) > 0.3)
        got = orc.pool_protect(raw, 4, 5)
        want = torch.nn.functional.max_pool1d(torch.from_numpy(raw)[:, None, :], 5, 1, 2)[:, 0].numpy()
        if not (np.array_equal(got[:, :-4], want[:, :-4]) and np.all(np.isinf(got[:, -4:]))):
            return False
        s = rng.integers(0, 4, size=(2, 30)).astype(np.float64)
        if not np.array_equal(orc.select(s, 11), brute.sort_select(s, 11)):
            return False
        qa = wl.bf16_bits(rng.standard_normal((4, 3, 8), dtype=np.float32) * 2)
        if not np.allclose(orc.attention_raw(qa, k), brute.attention_raw(qa, k), rtol=1e-12, atol=0):
            return False
        # in-place compaction with chains of moves, against fancy indexing
        c = wl.bf16_bits(rng.standard_normal((2, 9, 8), dtype=np.float32))
        kp = np.array([[1, 3, 4, 6], [0, 2, 5, 8]], dtype=np.int32)
        want = np.stack([c[g][kp[g]] for g in range(2)])
        if not np.array_equal(orc.compact_inplace(c.copy(), kp, 9)[:, :4], want):
            return False
        # rescoring a resident cache (finite garbage past n_valid) = scoring its valid rows
        kc = wl.bf16_bits(rng.standard_normal((2, 23, 8), dtype=np.float32))
        vc = wl.bf16_bits(rng.standard_normal((2, 23, 8), dtype=np.float32))
        want = orc.score(q, np.ascontiguousarray(kc[:, :17]), np.ascontiguousarray(vc[:, :17]), 3)
        if not np.array_equal(orc.rescore(q, kc, vc, 17, 3), want):
            return False
        return True
    except orc.OracleError:
        return False
    finally:
        orc._lib = saved


def test_unmutated_oracle_passes_the_compact_pins():
    assert _pins_pass(orc.lib())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(orc.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"liboracle_{name}.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(path),
                           "-o", so, "-lm"])
    assert not _pins_pass(orc.load(so)), f"planted mistake {name} went unnoticed"
