#!/usr/bin/env python3
"""Benchmark of the DropKV eviction path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = the whole path over one synthetic single-layer batch:
dropkv_score (pass 1, merge, pass 2 with pooling/protection)
-> dropkv_select -> dropkv_compact, with the inputs already resident in HBM.
The workload is the Llama-3.1-8B-shaped layer at n = 131072 (Hq=32, Hkv=8,
d=128, w=8, pool 7, 5 % budget), bf16 inputs drawn by the seeded generator.

Prints ONE JSON line on stdout; everything else goes to stderr.

Also:
  --summarize-pmc FETCH.csv WRITE.csv [FETCH_CMD WRITE_CMD]
                                        turn two rocprofv3 --pmc runs (FETCH_SIZE,
                                        WRITE_SIZE) into profiles/traffic_<workload>.json
  --copy-calibration                    run one 1 GiB device-to-device copy after the
                                        timed steps (the counters' scale reference)
  --summarize-util CSV COMMAND          rocprofv3 --pmc VALUBusy MfmaUtil output ->
                                        profiles/util_<workload>.txt
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["attention_perturbation_scoring_amd/csrc/common.h",
                  "attention_perturbation_scoring_amd/csrc/score_kernels.hip",
                  "attention_perturbation_scoring_amd/csrc/select_compact.hip",
                  "attention_perturbation_scoring_amd/csrc/measure.hip"]
COPY_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Algorithmic HBM bytes per (token, KV head) of each kernel; the whole score +
# select path moves 8d + 8 bytes per (token, KV head): two bf16 reads of K and V,
# one fp32 score write and one fp32 score read.
def algorithmic_bytes(kernel: str, Hkv: int, n: int, d: int, budget: int) -> float:
    th = Hkv * n
    if kernel == "pass1":
        return th * 4.0 * d
    if kernel == "pass2":
        return th * (4.0 * d + 4.0)
    if kernel == "select":
        return th * 4.0
    if kernel == "compact":
        return 2.0 * 2.0 * Hkv * budget * d * 2.0
    return 0.0


def traffic_for(workload: str, kernel: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None  # counters were taken on different kernels
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def time_layer_select(ctx, scores, Hkv, n, budget, stream, args):
    """Mean HIP-event time of dropkv_select_layer (same total budget as the
    per-head selection) over the scores of the last step."""
    import torch
    keep_l = torch.empty((Hkv * budget,), dtype=torch.int32, device="cuda")
    counts_l = torch.empty((Hkv,), dtype=torch.int32, device="cuda")
    for _ in range(args.warmup):
        ctx.select_layer(scores, Hkv, n, Hkv * budget, keep_l, counts_l, stream)
    ctx.profile(True)
    ctx.profile_reset()
    for _ in range(args.steps):
        ctx.select_layer(scores, Hkv, n, Hkv * budget, keep_l, counts_l, stream)
    torch.cuda.synchronize()
    tot, cnt = ctx.profile_read("select")   # selection + per-head counts: two scopes per call
    ctx.profile(False)
    ctx.check(stream)
    return 1e3 * tot / max(cnt // 2, 1)


def plant_peaked_key(cfg, inp, pstar=0.9999):
    """The layer's K with one key per KV head set so that every window row of
    the head puts probability ~pstar on it: for head g, the least-squares (here
    exact, G*w < d) solution b of Q_g b = ln(pstar (n-1) / (1-pstar)) sqrt(d),
    rounded to bf16, at a token every window row sees.  Rows whose arg-max
    holds more than ~0.94 take the exact exclusion fixup.  Returns the bf16
    bits of K and the planted token."""
    import math
    import numpy as np
    from attention_perturbation_scoring_amd import workload as wl
    G, d, n, w = cfg.Hq // cfg.Hkv, cfg.d, cfg.n, cfg.w
    q = wl.bf16_to_f32(inp["q"]).astype(np.float64)
    k = inp["k"].copy()
    jp = min(5000, n - w - 1)
    logit = math.log(pstar * (n - 1) / (1.0 - pstar)) * math.sqrt(d)
    for g in range(cfg.Hkv):
        Q = q[g * G:(g + 1) * G].reshape(-1, d)
        b, *_ = np.linalg.lstsq(Q, np.full(Q.shape[0], logit), rcond=None)
        k[g, jp] = wl.bf16_bits(b.astype(np.float32))
    return k, jp


def time_peaked_rows(ctx, cfg, inp, dev, v_dev, scores, stream):
    """Per-kernel HIP-event times of dropkv_score on the layer with a peaked
    key planted in every KV head (every window row takes the fixup)."""
    import torch
    from attention_perturbation_scoring_amd import dropkv
    k, jp = plant_peaked_key(cfg, inp)
    qd, kd = dev(inp["q"]), dev(k)
    Hq, Hkv, d, n, w, pool = cfg.Hq, cfg.Hkv, cfg.d, cfg.n, cfg.w, cfg.pool
    ctx.score(qd, kd, v_dev, n, w, Hq, Hkv, d, pool, scores, stream)
    status = ctx.sync(stream)
    if status != dropkv.OK:
        raise SystemExit(f"peaked rows: device status {dropkv.strerror(status)}")
    ctx.profile(True)
    ctx.profile_reset()
    for _ in range(3):
        ctx.score(qd, kd, v_dev, n, w, Hq, Hkv, d, pool, scores, stream)
    torch.cuda.synchronize()
    us = {}
    for name in ("pass1", "merge", "pass2"):
        tot, cnt = ctx.profile_read(name)
        if cnt:
            us[name] = round(1e3 * tot / cnt, 2)
    ctx.profile(False)
    ctx.check(stream)
    return {"what": "dropkv_score with every window row's arg-max planted at p* > 0.94 "
                    "(exact exclusion fixup on every row)",
            "planted_token": jp, "kernel_us": us}


def time_sink_heavy(ctx, cfg, dev, scores, keep, stream, steps):
    """Per-kernel HIP-event times of score + select on the sink-heavy variant of
    the workload (same shapes; every window row puts more than 0.94 of its
    attention on token 0, so every row takes the exact exclusion fixup), or
    None when the workload has no such variant."""
    import torch
    from attention_perturbation_scoring_amd import dropkv, workload as wl
    sc = wl.CONFIGS.get(cfg.name + "_sink")
    if sc is None:
        return None
    inp = wl.make_layer(sc, sc.seed)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    del inp
    Hq, Hkv, d, n, w, pool, budget = sc.Hq, sc.Hkv, sc.d, sc.n, sc.w, sc.pool, sc.budget

    def call():
        ctx.score_select(q, k, v, n, w, Hq, Hkv, d, pool, budget, scores, keep, stream)

    call()
    status = ctx.sync(stream)
    if status != dropkv.OK:
        raise SystemExit(f"sink-heavy: device status {dropkv.strerror(status)}")
    ctx.profile(True)
    ctx.profile_reset()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    us = {}
    for name in ("pass1", "merge", "pass2", "select"):
        tot, cnt = ctx.profile_read(name)
        if cnt:
            us[name] = round(1e3 * tot / cnt, 2)
    ctx.profile(False)
    ctx.check(stream)
    return {"workload": sc.name,
            "what": "score + select with every window row's arg-max (token 0) above 0.94 "
                    "of its attention (exact exclusion fixup on every row)",
            "kernel_us": us, "score_select_us": round(sum(us.values()), 2)}


def time_decode(ctx, cfg, q0, k0, v0, stream, steps, m=1024):
    """Decode-time pieces at the workload's shapes, on clones of the layer:
    (1) dropkv_compact_inplace of the whole prefill cache (capacity n) to the
    budget, with the prefill's own keep list; (2) dropkv_rescore of a resident
    cache whose first `budget` rows are survivors and whose next m rows stand
    for the decode tokens appended since: n_valid = budget + m rows are scored,
    `budget` of them kept, and the cache compacted in place."""
    import torch
    from attention_perturbation_scoring_amd import dropkv
    Hq, Hkv, d, n, w, pool, budget = cfg.Hq, cfg.Hkv, cfg.d, cfg.n, cfg.w, cfg.pool, cfg.budget
    if budget + m > n:
        return None
    k, v = k0.clone(), v0.clone()
    scores = torch.empty((Hkv, n), dtype=torch.float32, device="cuda")
    keep = torch.empty((Hkv, budget), dtype=torch.int32, device="cuda")
    ctx.score(q0, k, v, n, w, Hq, Hkv, d, pool, scores, stream)
    ctx.select(scores, Hkv, n, budget, keep, stream)
    ctx.check(stream)

    def kernel_avgs(names):
        out = {}
        for name in names:
            tot, cnt = ctx.profile_read(name)
            if cnt:
                out[name] = round(1e3 * tot / cnt, 2)
        return out

    # (1) the same ascending list applied again each time: the same moves, over
    # whatever the rows then hold
    ctx.compact_inplace(k, v, Hkv, n, n, d, keep, budget, stream)
    ctx.profile(True)
    ctx.profile_reset()
    for _ in range(steps):
        ctx.compact_inplace(k, v, Hkv, n, n, d, keep, budget, stream)
    torch.cuda.synchronize()
    inplace = kernel_avgs(["compact_inplace"])
    ctx.profile(False)
    ctx.check(stream)
    # (2) rescoring budget + m resident rows
    n_valid = budget + m
    sc2 = torch.empty((Hkv, n_valid), dtype=torch.float32, device="cuda")
    for _ in range(3):
        ctx.rescore(q0, k, v, n, n_valid, w, Hq, Hkv, d, pool, budget, sc2, keep, stream)
    ctx.check(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ctx.rescore(q0, k, v, n, n_valid, w, Hq, Hkv, d, pool, budget, sc2, keep, stream)
    torch.cuda.synchronize()
    call_us = (time.perf_counter() - t0) * 1e6 / steps
    ctx.profile(True)
    ctx.profile_reset()
    for _ in range(steps):
        ctx.rescore(q0, k, v, n, n_valid, w, Hq, Hkv, d, pool, budget, sc2, keep, stream)
    torch.cuda.synchronize()
    rk = kernel_avgs(["pass1", "merge", "pass2", "select", "compact_inplace"])
    ctx.profile(False)
    ctx.check(stream)
    del k, v
    return {"compact_inplace_full_us": inplace.get("compact_inplace"),
            "compact_inplace_what": f"{Hkv} heads x {budget} kept rows of a {n}-row cache, in place",
            "rescore": {"cap": n, "n_valid": n_valid, "m": m, "budget": budget,
                        "what": "dropkv_rescore: score the n_valid resident rows (window = last w), "
                                "keep budget, compact in place",
                        "call_us": call_us, "kernel_us": rk}}


def scratch_report(n, w, Hq, Hkv, d):
    """Device scratch the library holds for one call of these sizes, beside the
    pages' figures for the same question (n = 128K: ~17 MB for the fused Triton
    scorer against ~9 GB for the naive PyTorch one)."""
    from attention_perturbation_scoring_amd import dropkv
    sb, selb = dropkv.scratch_bytes(n, w, Hq, Hkv, d)
    return {"score": sb, "select": selb, "total": sb + selb,
            "what": "context scratch of dropkv_score (split partial states, per-row state) "
                    "and dropkv_select (histograms, candidates, per-block counts); no "
                    "attention weights or distances are materialised"}


def host_cpu() -> str:
    """The host's CPU model and logical CPU count, for the baseline's description."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, nproc {os.cpu_count()}"


def host_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, at most 16 (one
    GPU's share of the host)."""
    from oracle import oracle as orc
    return min(orc.default_threads(), 16)


def cpu_baseline(cfg, inp, dev_inputs):
    """Time the float64 oracle (score + select) on the host, on every host
    thread (the oracle spreads a call over all window rows of all KV heads):
    the full layer of a single-layer workload; for a multi-layer cache, the
    first KV heads of layer 0, projected to the whole cache."""
    import numpy as np
    from oracle import oracle as orc
    threads = host_threads()
    if cfg.layers > 1:
        q, k, v = dev_inputs
        G = cfg.Hq // cfg.Hkv
        heads = min(cfg.Hkv, threads)
        qs = q[: heads * G].cpu().numpy().view(np.uint16)
        ks = k[:heads].cpu().numpy().view(np.uint16)
        vs = v[:heads].cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        s = orc.score(qs, ks, vs, cfg.pool, nthreads=threads)
        orc.select(s, cfg.budget)
        dt = time.perf_counter() - t0
        whole = dt * (cfg.layers * cfg.Hkv) / heads
        return {"value": cfg.layers * cfg.n / whole, "unit": "tokens/s", "cores": threads,
                "kind": "oracle",
                "sample": f"{heads} KV heads of layer 0 of {cfg.name} (n={cfg.n}), float64 score + "
                          f"select in {dt:.2f} s on {threads} threads ({host_cpu()}), projected "
                          f"to all {cfg.layers * cfg.Hkv} heads"}
    t0 = time.perf_counter()
    s = orc.score(inp["q"], inp["k"], inp["v"], cfg.pool, nthreads=threads)
    orc.select(s, cfg.budget)
    dt = time.perf_counter() - t0
    # the per-core rate: one KV head on one thread, scaled to the layer
    t1 = time.perf_counter()
    G = cfg.Hq // cfg.Hkv
    s1 = orc.score(inp["q"][:G], inp["k"][:1], inp["v"][:1], cfg.pool, nthreads=1)
    orc.select(s1, cfg.budget)
    dt1 = (time.perf_counter() - t1) * cfg.Hkv
    return {"value": cfg.n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "value_one_thread": cfg.n / dt1,
            "sample": f"full {cfg.name} layer (all {cfg.Hkv} KV heads, n={cfg.n}); "
                      f"float64 score + select, {dt:.2f} s wall on {threads} threads "
                      f"(spread over the layer's {cfg.Hq * cfg.w} window rows; {host_cpu()}); "
                      f"one thread: KV head 0 alone, {dt1 / cfg.Hkv:.2f} s, scaled to the layer"}


def run(args):
    import numpy as np
    import torch
    from attention_perturbation_scoring_amd import dropkv, workload as wl

    cfg = wl.CONFIGS[args.workload]
    torch.cuda.set_device(0)
    L = cfg.layers

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")

    if L == 1:
        log(f"[bench] generating {cfg.name} inputs (seed {cfg.seed})")
        inp = wl.make_layer(cfg, cfg.seed)
        # Consecutive steps score different copies of the layer (different
        # addresses), as a multi-layer run scores a different layer each time: a
        # step never finds the previous step's reads still in the last-level cache.
        q0, k0, v0 = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
        copies = [(q0, k0, v0)] + [(q0.clone(), k0.clone(), v0.clone())
                                   for _ in range(args.rotate - 1)]
    else:
        # the full multi-layer cache, drawn on the device and folded into heads; it
        # is far larger than the last-level cache, so one copy suffices
        from attention_perturbation_scoring_amd import workload_device as wd
        log(f"[bench] drawing the {cfg.name} cache on the device ({L} layers)")
        inp = None
        copies = [wd.make_cache(cfg)]
        torch.cuda.synchronize()
    Hq, Hkv, d, n, w, pool, budget = (L * cfg.Hq, L * cfg.Hkv, cfg.d, cfg.n, cfg.w, cfg.pool,
                                      cfg.budget)
    scores = torch.empty((Hkv, n), dtype=torch.float32, device="cuda")
    keep = torch.empty((Hkv, budget), dtype=torch.int32, device="cuda")
    k_out = torch.empty((Hkv, budget, d), dtype=torch.int16, device="cuda")
    v_out = torch.empty((Hkv, budget, d), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    ctx = dropkv.Context(0)

    counter = [0]

    separate = getattr(args, "separate_calls", False)

    def score_select(q, k, v):
        if separate:
            ctx.score(q, k, v, n, w, Hq, Hkv, d, pool, scores, stream)
            ctx.select(scores, Hkv, n, budget, keep, stream)
        else:   # one call: the selection's first digit is counted in the second pass
            ctx.score_select(q, k, v, n, w, Hq, Hkv, d, pool, budget, scores, keep, stream)

    def step():
        q, k, v = copies[counter[0] % len(copies)]
        counter[0] += 1
        score_select(q, k, v)
        ctx.compact(k, v, Hkv, n, d, keep, budget, k_out, v_out, stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    ctx.check(stream)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ----
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    status = ctx.sync(stream)
    if status != dropkv.OK:
        raise SystemExit(f"device status {dropkv.strerror(status)}")
    ms_per_step = wall * 1e3 / args.steps

    # ---- per-kernel HIP-event timing over K more steps on the same stream ----
    ctx.profile(True)
    ctx.profile_reset()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof_wall = time.perf_counter() - t1
    kern = {}
    for name in dropkv.KERNELS:
        tot, cnt = ctx.profile_read(name)
        if cnt:
            kern[name] = {"avg_us": 1e3 * tot / cnt, "launches": cnt}
    ctx.profile(False)
    ctx.check(stream)

    # ---- the attention-only (SnapKV-style) score mode, timed the same way ----
    def attn_step():
        q, k, v = copies[counter[0] % len(copies)]
        counter[0] += 1
        ctx.score_attention(q, k, n, w, Hq, Hkv, d, pool, scores, stream)
        ctx.select(scores, Hkv, n, budget, keep, stream)
        ctx.compact(k, v, Hkv, n, d, keep, budget, k_out, v_out, stream)

    for _ in range(args.warmup):
        attn_step()
    ctx.check(stream)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        attn_step()
    torch.cuda.synchronize()
    attn_ms = (time.perf_counter() - t2) * 1e3 / args.steps
    ctx.profile(True)
    ctx.profile_reset()
    for _ in range(args.steps):
        attn_step()
    torch.cuda.synchronize()
    attn_kern = {}
    for name in ("attn_pass1", "attn_pass2", "select", "compact"):
        tot, cnt = ctx.profile_read(name)
        if cnt:
            attn_kern[name] = round(1e3 * tot / cnt, 2)
    ctx.profile(False)
    ctx.check(stream)
    attn_ss = sum(attn_kern.get(x, 0.0) for x in ("attn_pass1", "attn_pass2", "select"))
    attention_mode = {
        "what": "attention-only (SnapKV-style) scores + the same select + compact",
        "ms_per_step": attn_ms,
        "tokens_per_s": L * n / (attn_ms * 1e-3),
        "kernel_us": attn_kern,
        "score_select_us": attn_ss,
        # K read twice + score write/read: 4d + 8 bytes per (token, KV head)
        "score_select_algorithmic_GBs": Hkv * n * (4.0 * d + 8.0) / (attn_ss * 1e-6) / 1e9,
    }

    # ---- layer-wide selection (cross-head budgets) over the same scores ----
    layer_select_us = None
    if L == 1:
        layer_select_us = time_layer_select(ctx, scores, Hkv, n, budget, stream, args)

    # ---- the same layer with every window row peaked (the exclusion fixup) ----
    peaked_rows = sink_heavy = None
    if L == 1:
        log("[bench] peaked rows")
        peaked_rows = time_peaked_rows(ctx, cfg, inp, dev, copies[0][2], scores, stream)
        log("[bench] sink-heavy variant")
        sink_heavy = time_sink_heavy(ctx, cfg, dev, scores, keep, stream, max(3, min(args.steps, 10)))

    # ---- decode-time rescoring and in-place compaction ----
    decode = None
    if L == 1:
        log("[bench] decode-time rescoring")
        decode = time_decode(ctx, cfg, *copies[0], stream, max(3, min(args.steps, 20)))

    # ---- per-call distribution with the caches flushed before every call ----
    # Streaming 1 GiB through the caches evicts the 4 MB L2s and the 256 MB
    # last-level cache, so each call starts cold.  A read flush leaves clean
    # lines behind; a write flush (the fill) leaves up to the last-level
    # cache's size in dirty lines, whose write-back then lands inside the timed
    # call.  HIP events on the launch stream bracket score + select and
    # compaction separately.
    flush = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    flush.fill_(1.0)

    def cold_calls(how):
        ss_us, cp_us = [], []
        for i in range(args.steps):
            q, k, v = copies[i % len(copies)]
            if how == "read":
                ctx.stream_read(flush, stream=stream)
            else:
                flush.fill_(float(i))
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
            score_select(q, k, v)
            ev[1].record(stream)
            ctx.compact(k, v, Hkv, n, d, keep, budget, k_out, v_out, stream)
            ev[2].record(stream)
            ev[2].synchronize()
            ss_us.append(1e3 * ev[0].elapsed_time(ev[1]))
            cp_us.append(1e3 * ev[1].elapsed_time(ev[2]))
        ctx.check(stream)
        dist = lambda x: {"median": float(np.median(x)), "min": float(min(x)),
                          "p90": float(np.percentile(x, 90))}
        return {"score_select_us": dist(ss_us), "compact_us": dist(cp_us), "calls": args.steps}

    cold = {"read_flush": cold_calls("read"), "write_flush": cold_calls("write")}

    # ---- achievable read bandwidth: one streaming scan of the 1 GiB buffer ----
    for _ in range(3):
        ctx.stream_read(flush, stream=stream)
    ctx.profile(True)
    ctx.profile_reset()
    for _ in range(10):
        ctx.stream_read(flush, stream=stream)
    torch.cuda.synchronize()
    tot, cnt = ctx.profile_read("stream_read")
    ctx.profile(False)
    ctx.check(stream)
    achievable_gbs = COPY_BYTES / (1e-3 * tot / cnt) / 1e9
    del flush

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {COPY_BYTES} bytes done")

    score_select_us = sum(kern[x]["avg_us"] for x in ("pass1", "merge", "pass2", "select")
                          if x in kern)
    dom = max(("pass1", "pass2"), key=lambda x: kern[x]["avg_us"])
    alg = algorithmic_bytes(dom, Hkv, n, d, budget)
    achieved = alg / (kern[dom]["avg_us"] * 1e-6) / 1e9
    path_bytes = Hkv * n * (8.0 * d + 8.0)
    path_gbs = path_bytes / (score_select_us * 1e-6) / 1e9
    traffic = traffic_for(cfg.name, dom)

    out = {
        "metric": "KV tokens scored/s + achieved HBM GB/s (% of peak), n=128K, Hkv=8, d=128, w=8",
        "value": L * n / (ms_per_step * 1e-3),   # tokens (all layers) scored per second
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "Hq": Hq, "Hkv": Hkv, "d": d, "n": n, "w": w,
                   "pool": pool, "budget": budget, "batch": 1, "layers": L,
                   "input_dtype": "bf16", "step": "score+select+compact",
                   "calls": "dropkv_score + dropkv_select + dropkv_compact" if separate
                            else "dropkv_score_select + dropkv_compact",
                   "layer_copies": len(copies)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "kernel_us": {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()},
        "score_select_us": score_select_us,
        "score_select_algorithmic_GBs": path_gbs,
        "score_select_frac_of_peak": path_gbs / HBM_PEAK_GBS,
        "cold_cache_calls": cold,
        "achievable_read_GBs": achievable_gbs,
        "dominant_frac_of_achievable": achieved / achievable_gbs,
        "score_select_frac_of_achievable": path_gbs / achievable_gbs,
        "token_heads_per_s": Hkv * n / (ms_per_step * 1e-3),
        "profiled_ms_per_step": prof_wall * 1e3 / args.steps,
        "attention_mode": attention_mode,
        "layer_select_us": layer_select_us,
        "peaked_rows": peaked_rows,
        "sink_heavy": sink_heavy,
        "decode": decode,
        "kernel_source_hash": kernel_source_hash(),
        "scratch_bytes": scratch_report(n, w, Hq, Hkv, d),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, copies[0])
    ctx.close()
    return out


def summarize_pmc(fetch_csv: str, write_csv: str, workload: str, commands=()):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) from rocprofv3 counter CSVs,
    scaled by the same counters on the 1 GiB calibration copy.

    Each kernel family is averaged over the dispatches of the K timed steps
    only (from the pass-1 launch that opens step W to the compaction that
    closes step W + K - 1, in dispatch order; K and W read from the counter
    run's command), so the peaked-row, sink-heavy, decode-time and cold-cache
    calls the same run makes later do not enter the common path's figures; the
    attention-only kernels, which run only in their own mode, are averaged over
    all their dispatches.  The per-family means over every dispatch are kept
    beside them (`all_dispatches`)."""
    import re

    def load(path, counter):
        rows = []
        files = sorted(glob.glob(path)) if any(c in path for c in "*?[") else [path]
        for p in files:
            with open(p) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") != counter:
                        continue
                    key = r.get("Dispatch_Id") or r.get("Correlation_Id") or "0"
                    rows.append((int(key), r.get("Kernel_Name", ""), float(r["Counter_Value"])))
        rows.sort()
        return rows

    fetch = load(fetch_csv, "FETCH_SIZE")
    write = load(write_csv, "WRITE_SIZE")

    def matches(name, key):
        # "dropkv::pass1_kernel<" must not match "dropkv::attn_pass1_kernel<"
        return key in name if key == "copyBuffer" else f"::{key}" in name

    def window(rows, command):
        """(first, last) dispatch ids of the timed steps, or None."""
        m_s, m_w = re.search(r"--steps (\d+)", command or ""), re.search(r"--warmup (\d+)", command or "")
        if not (m_s and m_w):
            return None
        steps, warm = int(m_s.group(1)), int(m_w.group(1))
        p1 = [i for i, name, _ in rows if matches(name, "pass1_kernel")]
        if len(p1) < warm + steps:
            return None
        lo, last_p1 = p1[warm], p1[warm + steps - 1]
        comp = [i for i, name, _ in rows if matches(name, "compact_kernel") and i > last_p1]
        return (lo, comp[0]) if comp else None

    def mean(rows, key, win):
        vals = [v for i, name, v in rows if matches(name, key) and (win is None or win[0] <= i <= win[1])]
        return sum(vals) / len(vals) if vals else None

    cmds = list(commands) + [None, None]
    wf, ww = window(fetch, cmds[0]), window(write, cmds[1])
    # the calibration copy is the runtime's device-to-device blit of COPY_BYTES,
    # the largest copyBuffer dispatch of the run (the others are small uploads)
    cf = [v for _, name, v in fetch if matches(name, "copyBuffer")]
    cw = [v for _, name, v in write if matches(name, "copyBuffer")]
    copy_fetch, copy_write = (max(cf) if cf else None), (max(cw) if cw else None)
    f_scale = COPY_BYTES / (copy_fetch * 1024.0) if copy_fetch else None
    w_scale = COPY_BYTES / (copy_write * 1024.0) if copy_write else None
    # selection is one kernel when the head teams fit on the device, else four
    sel = ("select_fused",) if mean(fetch, "select_fused", None) is not None else (
        "select_s1", "select_s2", "select_s3", "select_s4")
    families = (("pass1", ("pass1_kernel",), True), ("merge", ("merge_kernel",), True),
                ("pass2", ("pass2_kernel",), True), ("select", sel, True),
                ("compact", ("compact_kernel",), True),
                ("attn_pass1", ("attn_pass1_kernel",), False),
                ("attn_pass2", ("attn_pass2_kernel",), False),
                ("compact_inplace", ("compact_inplace_kernel",), False))

    def family(keys, win_f, win_w):
        # a family of several kernels launched once each per call: sum per-launch means
        fks = [mean(fetch, k, win_f) for k in keys]
        wks = [mean(write, k, win_w) for k in keys]
        if None in fks or None in wks or f_scale is None or w_scale is None:
            return None
        fk, wk = sum(fks), sum(wks)
        return {"fetch_kib": fk, "write_kib": wk,
                "bytes_per_launch": fk * 1024.0 * f_scale + wk * 1024.0 * w_scale}

    kernels, everything = {}, {}
    for short, keys, timed in families:
        k_ = family(keys, wf if timed else None, ww if timed else None)
        if k_ is not None:
            kernels[short] = k_
        a_ = family(keys, None, None)
        if a_ is not None:
            everything[short] = a_
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": copy_fetch, "copy_write_kib": copy_write,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "window": {"fetch_dispatches": wf, "write_dispatches": ww,
                      "what": "the timed steps of the counter runs (common-path calls only)"},
           "kernels": kernels, "all_dispatches": everything,
           "counter_runs": list(commands),
           "made_by": f"python bench.py --summarize-pmc {fetch_csv} {write_csv} ..."}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    log(f"[bench] wrote {path}")


def summarize_util(csv_glob: str, workload: str, command: str):
    """rocprofv3 --pmc VALUBusy MfmaUtil CSV -> profiles/util_<workload>.txt:
    per kernel, the mean over dispatches of the percentage of the dispatch's
    GPU time the vector ALUs and the matrix cores were busy."""
    files = sorted(glob.glob(csv_glob)) if any(c in csv_glob for c in "*?[") else [csv_glob]
    vals = {}
    for p in files:
        with open(p) as f:
            for r in csv.DictReader(f):
                name = _short_name(r.get("Kernel_Name", ""))
                vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    lines = [f"rocprofv3 VALUBusy / MfmaUtil per dispatch, workload {workload}",
             f"kernel sources sha256[:16] {kernel_source_hash()}",
             f"command: {command}", "",
             f"{'kernel':<40}{'dispatches':>11}{'VALUBusy%':>11}{'MfmaUtil%':>11}"]
    for name, c in sorted(vals.items()):
        vb, mu = c.get("VALUBusy", []), c.get("MfmaUtil", [])
        nd = max(len(vb), len(mu))
        fmt = lambda xs: f"{sum(xs) / len(xs):>11.1f}" if xs else f"{'-':>11}"
        lines.append(f"{name[:39]:<40}{nd:>11}{fmt(vb)}{fmt(mu)}")
    path = os.path.join(ROOT, "profiles", f"util_{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"[bench] wrote {path}")


def _short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "").replace("dropkv::", "")


def summarize_kt(stats_csv: str, workload: str, command: str):
    """rocprofv3 --kernel-trace --stats CSV -> profiles/kernel_stats_<workload>.txt.

    The first table averages each kernel over the K timed steps and over the K
    event-profiled steps that follow them (the window between the pass-1
    launches that open those steps, read from the per-dispatch trace next to
    the statistics file); the second is rocprofv3's whole-run table, which
    also counts the warm-up, the cold-cache calls and the attention-only mode."""
    import re
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    steps = int(re.search(r"--steps (\d+)", command).group(1))
    warm = int(re.search(r"--warmup (\d+)", command).group(1))
    trace_csv = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    with open(trace_csv) as f:
        tr = [(_short_name(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
              for r in csv.DictReader(f)]
    tr.sort(key=lambda x: x[1])
    p1 = [t for t in tr if t[0].startswith("pass1_kernel")]
    lines = [f"rocprofv3 kernel statistics, workload {workload}",
             f"kernel sources sha256[:16] {kernel_source_hash()}",
             f"command: {command}", ""]
    for label, a, b in (("timed steps", warm, warm + steps),
                        ("event-profiled steps", warm + steps, warm + 2 * steps)):
        if len(p1) < b:
            continue
        # from the pass-1 launch opening step a to the end of the compaction
        # closing step b - 1
        lo = p1[a][1]
        hi = min(t[2] for t in tr if t[0].startswith("compact_kernel") and t[1] > p1[b - 1][1])
        per = {}
        for name, t0, t1 in tr:
            if lo <= t0 < hi and t1 <= hi:
                per.setdefault(name, []).append((t1 - t0) / 1e3)
        lines.append(f"{label} ({steps} steps, pass-1 launches {a}..{b - 1}):")
        lines.append(f"{'kernel':<34}{'calls':>7}{'avg_us':>11}{'min_us':>11}{'max_us':>11}")
        for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"{name[:33]:<34}{len(d):>7}{sum(d) / len(d):>11.2f}{min(d):>11.2f}"
                         f"{max(d):>11.2f}")
        lines.append("")
    lines.append("whole run (rocprofv3 --stats):")
    lines.append(f"{'kernel':<34}{'calls':>7}{'avg_us':>11}{'min_us':>11}{'max_us':>11}{'share%':>9}")
    for r in rows:
        lines.append(f"{_short_name(r['Name'])[:33]:<34}{int(r['Calls']):>7}"
                     f"{float(r['AverageNs']) / 1e3:>11.2f}"
                     f"{float(r['MinNs']) / 1e3:>11.2f}{float(r['MaxNs']) / 1e3:>11.2f}"
                     f"{float(r['Percentage']):>9.2f}")
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{workload}.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"[bench] wrote {path}")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=2,
                    help="copies of the layer that consecutive steps cycle through")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time dropkv_score + dropkv_select instead of dropkv_score_select")
    ap.add_argument("--summarize-pmc", nargs="+",
                    metavar="FETCH_CSV WRITE_CSV [FETCH_COMMAND WRITE_COMMAND]")
    ap.add_argument("--summarize-kt", nargs=2, metavar=("STATS_CSV", "COMMAND"))
    ap.add_argument("--summarize-util", nargs=2, metavar=("COUNTER_CSV", "COMMAND"))
    args = ap.parse_args()
    if args.summarize_util:
        summarize_util(args.summarize_util[0], args.workload, args.summarize_util[1])
        return
    if args.summarize_kt:
        summarize_kt(args.summarize_kt[0], args.workload, args.summarize_kt[1])
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      args.summarize_pmc[2:])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the DropKV path here runs on a single device "
              "(no inter-GPU collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    out = run(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
