"""bench.py's contract pieces that need no GPU: the one-GPU refusal, the
roofline's algorithmic byte accounting, and the counter-summary arithmetic."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line for a configuration that is not measured


@pytest.mark.parametrize("d", [8, 96, 128, 256])
def test_algorithmic_bytes_add_up_to_8d_plus_8_per_token_head(d):
    Hkv, n, budget = 8, 131072, 6553
    per = lambda k: bench.algorithmic_bytes(k, Hkv, n, d, budget) / (Hkv * n)
    # two bf16 reads of K and V, one fp32 score write (pass 2) and one read (select)
    assert per("pass1") + per("pass2") + per("select") == 8 * d + 8
    # compaction: K and V rows of the kept tokens, read once and written once
    assert bench.algorithmic_bytes("compact", Hkv, n, d, budget) == 2 * 2 * Hkv * budget * d * 2


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    # FETCH_SIZE counts half of what the calibration copy read, WRITE_SIZE all of it
    copy_kib = bench.COPY_BYTES / 1024
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", copy_kib / 2), ("__amd_rocclr_copyBuffer", 3.0),
        ("void dropkv::pass1_kernel<128, true>(dropkv::ScoreArgs)", 1000.0),
        ("void dropkv::pass1_kernel<128, true>(dropkv::ScoreArgs)", 1200.0),
        ("void dropkv::attn_pass1_kernel<128, true>(dropkv::ScoreArgs)", 50.0),
    ])
    _counter_csv(write, "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", copy_kib), ("__amd_rocclr_copyBuffer", 3.0),
        ("void dropkv::pass1_kernel<128, true>(dropkv::ScoreArgs)", 10.0),
        ("void dropkv::pass1_kernel<128, true>(dropkv::ScoreArgs)", 30.0),
        ("void dropkv::attn_pass1_kernel<128, true>(dropkv::ScoreArgs)", 5.0),
    ])
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "test")
    bench.summarize_pmc(str(fetch), str(write), "unit")
    with open(tmp_path / "profiles" / "traffic_unit.json") as f:
        t = json.load(f)
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    # pass 1: mean 1100 KiB fetched (x2) + mean 20 KiB written; the attention
    # kernel's name must not be mistaken for pass 1's
    assert t["kernels"]["pass1"]["bytes_per_launch"] == pytest.approx((2 * 1100 + 20) * 1024)
    assert t["kernels"]["attn_pass1"]["bytes_per_launch"] == pytest.approx((2 * 50 + 5) * 1024)


def test_traffic_summary_averages_the_timed_steps_only(tmp_path, monkeypatch):
    """The common path's per-launch figures come from the K timed steps (after W
    warm-up steps, read from the counter run's command); a later peaked-row
    merge stays out of them and is seen only in the all-dispatch means."""
    import csv as csv_
    seq = []
    for _ in range(5):   # 2 warm-up + 3 timed steps
        seq += [("void dropkv::pass1_kernel<128, true>(x)", 100.0), ("void dropkv::merge_kernel<128>(x)", 10.0),
                ("void dropkv::pass2_kernel<128, true, 4>(x)", 100.0), ("dropkv::select_fused(x)", 5.0),
                ("dropkv::compact_kernel(x)", 20.0)]
    seq += [("void dropkv::pass1_kernel<128, true>(x)", 100.0), ("void dropkv::merge_kernel<128>(x)", 999.0),
            ("void dropkv::pass2_kernel<128, true, 4>(x)", 100.0), ("__amd_rocclr_copyBuffer", 524288.0)]
    for path, counter in ((tmp_path / "f.csv", "FETCH_SIZE"), (tmp_path / "w.csv", "WRITE_SIZE")):
        with open(path, "w", newline="") as f:
            w = csv_.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for i, (name, v) in enumerate(seq, 1):
                if counter == "WRITE_SIZE" and "copyBuffer" in name:
                    v = 1048576.0
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "test")
    cmd = "rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --steps 3 --warmup 2"
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "unit", [cmd, cmd])
    with open(tmp_path / "profiles" / "traffic_unit.json") as f:
        t = json.load(f)
    assert t["window"]["fetch_dispatches"] == [11, 25]
    assert t["kernels"]["merge"]["fetch_kib"] == pytest.approx(10.0)
    assert t["all_dispatches"]["merge"]["fetch_kib"] > 10.0


@pytest.mark.parametrize("name", ["tiny", "llama4k"])
def test_planted_key_peaks_every_window_row(name):
    """The peaked-rows measurement's input: in every KV head the planted token
    is every window row's arg-max, at p* above the 0.94 fixup threshold."""
    import math
    import numpy as np
    from attention_perturbation_scoring_amd import workload as wl
    cfg = wl.CONFIGS[name]
    inp = wl.make_layer(cfg, cfg.seed)
    k, jp = bench.plant_peaked_key(cfg, inp)
    q = wl.bf16_to_f32(inp["q"]).astype(np.float64)
    kf = wl.bf16_to_f32(k).astype(np.float64)
    G, d, n, w = cfg.Hq // cfg.Hkv, cfg.d, cfg.n, cfg.w
    for h in range(cfg.Hq):
        logits = q[h] @ kf[h // G].T / math.sqrt(d)      # [w][n]
        for t in range(w):
            row = logits[t, : n - w + t + 1]             # the keys window query t sees
            p = np.exp(row - row.max())
            p /= p.sum()
            assert int(np.argmax(p)) == jp and p[jp] > 0.95, (name, h, t, p[jp])
    # only the planted token changed
    diff = np.argwhere(k != inp["k"])
    assert set(diff[:, 1].tolist()) <= {jp}
