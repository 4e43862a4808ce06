#!/usr/bin/env python3
"""Benchmark of DSA sparse attention (indexer -> top-k -> sparse MLA attention) on one MI355X.

Headline: decode throughput (query tokens/s, one query row per sequence) and
algorithmic HBM GB/s on the mixed-length workload (batch 64, contexts uniform in
[16384, 131072], top-k 2048, 128 heads over a 576/512 latent, indexer 64 x 128,
paged blocks of 64).  One step is one sparse_attn_decode call over the whole
batch: indexer scan, top-k, attention and split merge, with every input already
resident in HBM.  Secondary lines: prefill query-tokens/s on the L = 32768
workload, and the CPU oracle timed on the host cores on a bounded sample.

Per-kernel durations come from HIP events that the profiling entry point records
on the library's stream between its kernels, in event-marked steps of their own.
Order of a run: peak probe, the other decode workloads (batch 32 x 8K, 4 x 1M,
64 x 128K, each back to back and with a 1 GiB cache flush before every step),
the two prefill lines, the supplementary decode calls on the headline batch,
its event-marked and flushed steps, and last the headline: W warm-up steps,
then K plain steps between two synchronisations.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
TOPK_PATHS = {0: "default", 1: "threshold", 2: "onepass_u2", 3: "onepass_u4"}
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
METRIC = "decode tokens/s + HBM GB/s at 128K ctx, top-k=2048; prefill query-tokens/s"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_algorithmic(w):
    """Bytes and flops the method must move/do for one decode call (fp32 output)."""
    import numpy as np
    sh = w["shape"]
    ctx = w["context_lens"].astype(np.int64)
    kept = np.minimum(ctx, sh.topk)
    blocks = (ctx + sh.block_size - 1) // sh.block_size
    scan = int((ctx * sh.idx_dim * 2).sum())
    gather = int((kept * sh.qk_dim * 2).sum())
    per_q = sh.num_heads * sh.qk_dim * 2 + sh.num_heads * sh.v_dim * 4 + sh.num_heads * 4 + \
        sh.idx_heads * (2 * sh.idx_dim + 4)
    total = scan + gather + len(ctx) * per_q + int((4 * kept).sum()) + int((4 * blocks).sum())
    flops = int((2 * ctx * sh.idx_heads * sh.idx_dim).sum() + (2 * kept * sh.num_heads * (sh.qk_dim + sh.v_dim)).sum())
    # the indexer scan alone, as the method needs it: the key rows, the row's
    # indexer query and head weights, and one block-table entry per block (the
    # fp32 scores the scan writes for the top-k are not counted)
    idx_bytes = int((ctx * sh.idx_dim * 2).sum() + len(ctx) * sh.idx_heads * (2 * sh.idx_dim + 4) +
                    (4 * blocks).sum())
    # the attention alone: the kept latent rows, the queries and the outputs
    attn_bytes = gather + len(ctx) * sh.num_heads * (sh.qk_dim * 2 + sh.v_dim * 4)
    attn_flops = int((2 * kept * sh.num_heads * (sh.qk_dim + sh.v_dim)).sum())
    return dict(bytes=total, scan=scan, gather=gather, flops=flops, indexer_bytes=idx_bytes,
                attention_bytes=attn_bytes, attention_flops=attn_flops)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "dsa_sparse_attention_02_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key, launches_per_step):
    """HBM bytes per launch from the committed counter summary, or None if the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != source_hash(*e.get("sources", [])):
        return None
    return e.get("bytes_per_launch")


def setup_decode(name, torch, sa, synth):
    """Generate a decode workload, copy it to the device, and prepare the plain
    and event-marked calls over it."""
    spec = synth.WORKLOADS[name]
    log(f"generating {spec.name} (seed {spec.seed})")
    t = time.time()
    w = synth.make(spec)
    log(f"generated in {time.time() - t:.1f}s; copying to the device")
    d = sa.to_device(w)
    p = sa.Params.from_shape(w["shape"])
    B = spec.batch
    max_ctx = int(w["context_lens"].max())
    ws = torch.empty(sa.decode_workspace_size(p, B, max_ctx), dtype=torch.uint8, device="cuda")
    outs = sa._outputs(p, B, "cuda", True)
    marked = lambda ev: sa.sparse_attn_decode_profiled(p, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"], ev,
                                                       workspace=ws, outputs=outs)
    plain = lambda: sa.sparse_attn_decode(p, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"], workspace=ws,
                                          outputs=outs)
    n_marks = marked([])[3]
    kernels = (["indexer", "topk", "attention", "merge"] if max_ctx > p.topk else
               ["topk", "attention", "merge"])[:n_marks - 1]
    return dict(name=name, w=w, d=d, p=p, B=B, max_ctx=max_ctx, ws=ws, outs=outs, plain=plain, marked=marked,
                n_marks=n_marks, kernels=kernels, alg=decode_algorithmic(w))


def time_back_to_back(torch, fn, steps, warmup):
    """warmup untimed calls, then `steps` calls timed between two synchronisations (ms per call)"""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_stages(torch, sa, c, steps):
    """Per-kernel durations from HIP events that the profiling entry point
    records on the library's stream between its kernels; also the step time of
    these event-marked steps (an event between kernels delays the next one)."""
    events = [[sa.HipEvent() for _ in range(c["n_marks"])] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        c["marked"](events[s])
    torch.cuda.synchronize()
    ms_marked = (time.perf_counter() - t0) * 1e3 / steps
    per_kernel = {k: [ev[i].elapsed_ms(ev[i + 1]) for ev in events] for i, k in enumerate(c["kernels"])}
    return {k: statistics.mean(v) for k, v in per_kernel.items()}, ms_marked


def time_flushed(torch, sa, c, steps):
    """Steps with a 1 GiB write before each (the 256 MB MALL and the L2 hold
    none of the step's data), each timed alone between events; median ms."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    times = []
    for _ in range(steps):
        flush.fill_(1.0)
        ev = [sa.HipEvent() for _ in range(c["n_marks"])]
        c["marked"](ev)
        torch.cuda.synchronize()
        times.append(ev[0].elapsed_ms(ev[-1]))
    del flush
    return statistics.median(times), min(times)


def decode_line(c, ms):
    """tokens/s and algorithmic HBM rate of a decode step of ms milliseconds"""
    B, alg = c["B"], c["alg"]
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(B / (ms / 1e3), 1),
            "hbm_gbps": round(alg["bytes"] / (ms / 1e3) / 1e9, 1),
            "hbm_frac": round(alg["bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes_per_step": alg["bytes"]}


def supplementary_decode(args, torch, sa, synth, c):
    """On the headline batch: the call that appends each sequence's current
    token first, the run-time tuned call, and block-granular selection."""
    p, d, w, B, max_ctx, ws, outs = c["p"], c["d"], c["w"], c["B"], c["max_ctx"], c["ws"], c["outs"]
    res = {}
    if args.append_steps > 0:
        nk_np, ni_np = synth.new_tokens(w)
        nk = torch.from_numpy(nk_np).view(torch.bfloat16).cuda()
        ni = torch.from_numpy(ni_np).view(torch.bfloat16).cuda()
        # (the same token every step, so the cache keeps its values)
        app = lambda: sa.sparse_attn_decode_append(p, d["cache"], max_ctx, nk, ni, d["q"], d["idx_q"], d["idx_w"],
                                                   workspace=ws, outputs=outs)
        ms_app = time_back_to_back(torch, app, args.append_steps, 20)
        ms_plain = time_back_to_back(torch, c["plain"], args.append_steps, 0)
        log(f"decode with append: {ms_app:.3f} ms/step (plain step right after it: {ms_plain:.3f} ms)")
        res["decode_append"] = {"ms_per_step": round(ms_app, 4), "tokens_per_s": round(B / (ms_app / 1e3), 1),
                                "added_us": round((ms_app - ms_plain) * 1e3, 2)}
    if args.tune:
        splits, path, partners, tune_us = sa.decode_tune(p, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"],
                                                         reps=10)
        wst = torch.empty(sa.decode_workspace_size_cfg(p, B, max_ctx, splits, path), dtype=torch.uint8,
                          device="cuda")
        cfg = lambda: sa.sparse_attn_decode_cfg(p, d["cache"], max_ctx, splits, d["q"], d["idx_q"], d["idx_w"],
                                                topk_path=path, attn_partners=partners, workspace=wst, outputs=outs)
        ms = time_back_to_back(torch, cfg, 20, 20)
        log(f"tuned: {splits} attention splits per row, top-k path {TOPK_PATHS[path]}, attention partners "
            f"{partners or 'default'}, {ms:.3f} ms/step (tuner's own mean {tune_us:.1f} us)")
        res["decode_tuned"] = {"attn_splits": splits, "topk_path": TOPK_PATHS[path], "attn_partners": partners,
                               "ms_per_step": round(ms, 4), "tokens_per_s": round(B / (ms / 1e3), 1)}
        del wst
    if args.partners_steps > 0:
        # both attention kernels (two or four partner waves per head block),
        # interleaved over three rounds
        times = {2: [], 4: []}
        for _ in range(3):
            for n in times:
                f = lambda n=n: sa.sparse_attn_decode_cfg(p, d["cache"], max_ctx, 0, d["q"], d["idx_q"], d["idx_w"],
                                                          attn_partners=n, workspace=ws, outputs=outs)
                times[n].append(time_back_to_back(torch, f, args.partners_steps, 10))
        res["decode_partners"] = {f"{n}_partners_ms_per_step": round(sorted(v)[1], 4) for n, v in times.items()}
        log(f"attention kernels (median of 3 rounds): {res['decode_partners']}")
    if args.blocks_steps > 0:
        from dataclasses import replace
        sh = w["shape"]
        pb = sa.Params.from_shape(replace(sh, topk=sh.topk // sh.block_size))
        wsb = torch.empty(sa.decode_blocks_workspace_size(pb, B, max_ctx), dtype=torch.uint8, device="cuda")
        outb = sa._outputs(pb, B, "cuda", True)
        blk = lambda: sa.sparse_attn_decode_blocks(pb, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"],
                                                   workspace=wsb, outputs=outb)
        ms = time_back_to_back(torch, blk, args.blocks_steps, 20)
        log(f"decode with block selection ({pb.topk} blocks of {sh.block_size}): {ms:.3f} ms/step")
        res["decode_blocks"] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(B / (ms / 1e3), 1),
                                "kept_blocks": pb.topk, "block_size": sh.block_size}
        del wsb, outb
    return res


def run_other_decode(args, torch, sa, synth, name):
    """Another decode configuration: back-to-back steps, MALL-flushed steps
    (median) and per-kernel stages; supplementary lines, not the metric."""
    c = setup_decode(name, torch, sa, synth)
    ms = time_back_to_back(torch, c["plain"], 20, 50)
    stages, _ = time_stages(torch, sa, c, 10)
    cold, cold_min = time_flushed(torch, sa, c, 10)
    line = decode_line(c, ms)
    line["flushed"] = {"median_ms": round(cold, 4), "min_ms": round(cold_min, 4),
                       "tokens_per_s": round(c["B"] / (cold / 1e3), 1),
                       "hbm_frac": round(c["alg"]["bytes"] / (cold / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
    line["stages_us"] = {k: round(v * 1e3, 2) for k, v in stages.items()}
    log(f"{name}: {ms:.4f} ms/step back to back, {cold:.4f} ms flushed (median); stages " +
        ", ".join(f"{k} {v * 1e3:.1f}us" for k, v in stages.items()))
    if args.tune:
        p, d = c["p"], c["d"]
        splits, path, partners, _ = sa.decode_tune(p, d["cache"], c["max_ctx"], d["q"], d["idx_q"], d["idx_w"],
                                                   reps=10)
        wst = torch.empty(sa.decode_workspace_size_cfg(p, c["B"], c["max_ctx"], splits, path), dtype=torch.uint8,
                          device="cuda")
        cfg = lambda: sa.sparse_attn_decode_cfg(p, d["cache"], c["max_ctx"], splits, d["q"], d["idx_q"],
                                                d["idx_w"], topk_path=path, attn_partners=partners, workspace=wst,
                                                outputs=c["outs"])
        mt = time_back_to_back(torch, cfg, 20, 20)
        line["tuned"] = {"attn_splits": splits, "topk_path": TOPK_PATHS[path], "attn_partners": partners,
                         "ms_per_step": round(mt, 4), "tokens_per_s": round(c["B"] / (mt / 1e3), 1)}
    del c
    torch.cuda.empty_cache()
    return line


def prefill_pieces(w):
    """(first row, rows, first position) of every non-empty sequence of a prefill workload."""
    if w["mode"] == "varlen":
        cu, qs = w["cu_seqlens"], w["q_starts"]
        return [(int(cu[s]), int(cu[s + 1] - cu[s]), int(qs[s])) for s in range(len(qs)) if cu[s + 1] > cu[s]]
    return [(0, int(w["rows"]), int(w["q_start"]))]


def prefill_select_kernels(pieces, topk):
    """Kernel names of the select stage in launch order (mirrors the library's
    planning: chunks of rows whose fp32 scores take at most 1 GiB, in multiples
    of 16 rows, at most 64 pieces of one sequence per chunk; the indexer only
    where some row sees more than topk keys)."""
    total = sum(n for _, n, _ in pieces)
    stride = (max(q + n for _, n, q in pieces) + 63) // 64 * 64
    chunk = min(max(16, ((1 << 30) // (stride * 4)) // 16 * 16), (total + 15) // 16 * 16)
    names, r0 = [], 0
    while r0 < total:
        rmax, parts, r1 = min(total, r0 + chunk), [], r0
        for a, n, q in pieces:
            if a + n <= r0 or len(parts) == 64 or r1 >= rmax:
                continue
            lo, hi = max(r0, a), min(rmax, a + n)
            parts.append(q + hi - a)  # the last position in the chunk, + 1
            r1 = hi
        if any(e > topk for e in parts):
            names.append("indexer")
        names.append("topk")
        r0 = r1
    return names


def run_prefill(args, torch, sa, synth, name="prefill_L32k"):
    spec = synth.WORKLOADS[name]
    log(f"generating {spec.name}")
    w = synth.make(spec)
    d = sa.to_device(w)
    p = sa.Params.from_shape(w["shape"])
    L = int(w["rows"])
    outs = sa._outputs(p, L, "cuda", True)
    if w["mode"] == "varlen":
        ws = torch.empty(sa.prefill_varlen_workspace_size(p, w["cu_seqlens"], w["q_starts"]), dtype=torch.uint8,
                         device="cuda")
        call = lambda ev: sa.sparse_attn_prefill_varlen(p, d["cache"], w["cu_seqlens"], w["q_starts"], d["q"],
                                                        d["idx_q"], d["idx_w"], workspace=ws, outputs=outs,
                                                        events=ev)
    else:
        ws = torch.empty(sa.prefill_workspace_size(p, L, w["q_start"]), dtype=torch.uint8, device="cuda")
        call = lambda ev: sa.sparse_attn_prefill_profiled(p, d["cache"], w["q_start"], d["q"], d["idx_q"],
                                                          d["idx_w"], ev, workspace=ws, outputs=outs)
    n_marks = call([])[3]
    torch.cuda.synchronize()
    steps = max(1, args.prefill_steps)
    evs = [[sa.HipEvent() for _ in range(n_marks)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        call(evs[s])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # launch order: per chunk [indexer?, topk], then attention (+ merge)
    sh = w["shape"]
    pieces = prefill_pieces(w)
    names = prefill_select_kernels(pieces, p.topk)
    n_attn = n_marks - 1 - len(names)
    if n_attn < 1:
        raise SystemExit(f"prefill marks ({n_marks}) do not match the chunk plan ({len(names)} select kernels)")
    names += ["attention"] * n_attn
    tot = {}
    for ev in evs:
        for i, k in enumerate(names):
            tot[k] = tot.get(k, 0.0) + ev[i].elapsed_ms(ev[i + 1]) / steps
    # causal pairs: row i of a piece at position q + i sees q + i + 1 keys
    pairs = sum(n * q + n * (n + 1) // 2 for _, n, q in pieces)
    kept = sum(min(q + i + 1, sh.topk) for _, n, q in pieces for i in range(n))
    idx_flops = 2.0 * sh.idx_heads * sh.idx_dim * pairs
    attn_flops = 2.0 * sh.num_heads * (sh.qk_dim + sh.v_dim) * kept
    res = dict(workload=spec.name, ms_per_step=round(ms, 3), value=round(L / (ms / 1e3), 1), unit="query tokens/s",
               stages_ms={k: round(v, 3) for k, v in tot.items()},
               indexer_tflops=round(idx_flops / (tot.get("indexer", float("nan")) / 1e3) / 1e12, 1),
               attention_tflops=round(attn_flops / (tot["attention"] / 1e3) / 1e12, 1))
    res["indexer_mfma_frac"] = round(res["indexer_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
    res["attention_mfma_frac"] = round(res["attention_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
    # the same rows in plain calls under both schedules: every chunk's select,
    # then the attention (serial), or select and attention pipelined by chunk
    cu, qs = (w["cu_seqlens"], w["q_starts"]) if w["mode"] == "varlen" else ([0, L], [w["q_start"]])
    wsv = torch.empty(sa.prefill_varlen_workspace_size(p, cu, qs), dtype=torch.uint8, device="cuda")
    sched = {}
    for sname, code in (("serial", sa.SA_PREFILL_SERIAL), ("pipelined", sa.SA_PREFILL_PIPELINED)):
        f = lambda code=code: sa.sparse_attn_prefill_varlen(p, d["cache"], cu, qs, d["q"], d["idx_q"], d["idx_w"],
                                                            workspace=wsv, outputs=outs, pipeline=code)
        sched[sname] = round(time_back_to_back(torch, f, steps, 1), 3)
    res["schedules_ms_per_step"] = sched
    if args.partners_steps > 0:
        part = {}
        for n in (2, 4):
            f = lambda n=n: sa.sparse_attn_prefill_varlen(p, d["cache"], cu, qs, d["q"], d["idx_q"], d["idx_w"],
                                                          workspace=wsv, outputs=outs, attn_partners=n)
            part[f"{n}_partners"] = round(time_back_to_back(torch, f, steps, 1), 3)
        res["attention_partners_ms_per_step"] = part
    log(f"{spec.name}: {ms:.2f} ms/step, stages {res['stages_ms']}; plain calls {sched}")
    return res


def measured_peaks():
    """The peak probe (dsa_sparse_attention_02_amd/peak_probe, built with the
    library): streamed HBM read and copy rates, bf16 MFMA throughput and LDS
    read bandwidth of this GPU, or None when the probe is missing."""
    import subprocess
    exe = os.path.join(ROOT, "dsa_sparse_attention_02_amd", "peak_probe")
    if not os.path.exists(exe):
        log("peak probe not built; no measured peaks")
        return None
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        log(f"peak probe failed: {r.stderr.strip()[-200:]}")
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def cpu_model():
    """The host CPU's model name (as lscpu reports it, from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(args, w):
    """The oracle as it stands, on the host's cores, over a bounded sample of the
    same batch: rows longest first, passes repeated until the time budget is spent."""
    import oracle
    import numpy as np
    ctx = w["context_lens"]
    order = np.argsort(ctx)[::-1]  # start with the longest rows: the costliest per token
    done, distinct, t0 = 0, set(), time.perf_counter()
    stage = np.zeros(3)
    while time.perf_counter() - t0 < args.cpu_seconds:
        for r in order:
            oracle.run(w, rows=[int(r)], stage_seconds=stage)
            done += 1
            distinct.add(int(r))
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
    el = time.perf_counter() - t0
    rows = sorted(distinct)
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"{done} decode-row evaluations over {len(rows)} of {len(ctx)} rows of {args.workload} "
                      f"(longest first, ctx {int(ctx[rows].min())}-{int(ctx[rows].max())}, repeated to fill the "
                      f"budget); {el:.1f}s: indexer {stage[0]:.1f}s, sort {stage[1]:.1f}s, attention {stage[2]:.1f}s"}


TRAFFIC_KERNEL = "idx_score_decode_kernel<128, 2, true>"
TRAFFIC_SOURCES = ["indexer.hpp", "device_common.hpp"]


def _counter_rows(path):
    """(kernel name, counter name, value) of every row of a rocprofv3 counter CSV
    (a file, or a directory searched for *counter_collection.csv)."""
    import csv
    import glob
    files = [path] if os.path.isfile(path) else \
        glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                out.append((row["Kernel_Name"], row["Counter_Name"], float(row["Counter_Value"])))
    return out


def traffic_summary(fetch_path, write_path, workload):
    """HBM bytes per launch of the decode scan from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
    same counter reads for a plain 1 GiB device copy (bench.py --copy-calibration)."""
    def per_kernel(rows, counter):
        vals = {}
        for k, c, v in rows:
            if c == counter:
                vals.setdefault(k, []).append(v)
        return vals
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_path), ("WRITE_SIZE", write_path)):
        vals = per_kernel(_counter_rows(path), counter)
        kib = 1 << 20  # a 1 GiB copy reads and writes 1 GiB
        copies = [v for k, vs in vals.items() if "copy" in k.lower() or "elementwise" in k.lower()
                  for v in vs if 0.5 * kib < v < 4 * kib]
        if not copies:
            raise SystemExit(f"no 1 GiB copy dispatch found for {counter}")
        factor = kib / statistics.median(copies)
        scan = [v for k, vs in vals.items() if k.startswith("void sa::idx_score_decode_kernel<128, 2, true>")
                or k.startswith("sa::idx_score_decode_kernel<128, 2, true>") for v in vs]
        if not scan:
            raise SystemExit(f"no decode-scan dispatch found for {counter}")
        res[counter] = dict(kib_raw=statistics.median(scan), copy_kib_raw=statistics.median(copies),
                            factor=factor, bytes=statistics.median(scan) * factor * 1024, dispatches=len(scan))
    return {"kernel": TRAFFIC_KERNEL, "workload": workload, "sources": TRAFFIC_SOURCES,
            "source_hash": source_hash(*TRAFFIC_SOURCES),
            "fetch_bytes_per_launch": round(res["FETCH_SIZE"]["bytes"]),
            "write_bytes_per_launch": round(res["WRITE_SIZE"]["bytes"]),
            "bytes_per_launch": round(res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]),
            "counters": res}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first; tens of milliseconds of work can leave the clocks below their "
                         "loaded level, so the default warms up for about 0.1 s")
    ap.add_argument("--workload", default="decode_b64_ctx16k_128k")
    ap.add_argument("--flush-steps", type=int, default=10, help="extra steps timed after a 1 GiB cache flush")
    ap.add_argument("--prefill-steps", type=int, default=2)
    ap.add_argument("--append-steps", type=int, default=20,
                    help="steps of the decode call that also appends each sequence's current token to the "
                         "cache (sparse_attn_decode_append), timed like the plain steps right after them")
    ap.add_argument("--blocks-steps", type=int, default=20,
                    help="steps of block-granular decode (sparse_attn_decode_blocks, k / block_size blocks per "
                         "row) over the same batch")
    ap.add_argument("--no-tune", dest="tune", action="store_false",
                    help="skip the run-time tuning of the attention split count and top-k path (sa_decode_tune)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--partners-steps", type=int, default=20,
                    help="steps per round timing both attention kernels (two or four partner waves), 0 = skip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the HBM / MFMA / LDS peak probe")
    ap.add_argument("--other-workloads", default="decode_b32_ctx8k,decode_b4_ctx1m,decode_b64_ctx128k_full",
                    help="comma-separated decode workloads also timed (supplementary lines, not the metric; "
                         "'none' for the headline workload only)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) of this "
                         "benchmark into profiles/traffic.json")
    args = ap.parse_args()
    if args.traffic_from:
        t = traffic_summary(args.traffic_from[0], args.traffic_from[1], args.workload)
        path = os.path.join(ROOT, "profiles", "traffic.json")
        try:
            with open(path) as f:
                allt = json.load(f)
        except (OSError, ValueError):
            allt = {}
        allt[TRAFFIC_KERNEL + "/" + args.workload] = t
        with open(path, "w") as f:
            json.dump(allt, f, indent=1)
        print(json.dumps(t, indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the sparse-attention path here is single-GPU "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from dsa_sparse_attention_02_amd import sparse_attn as sa
    from dsa_sparse_attention_02_amd import synth
    sa.lib()  # fail loudly if the library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # an elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        log("copy calibration: 3 elementwise copies of 1 GiB")
        del src, dst

    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks()
        log(f"measured peaks: {peaks}")
    # The supplementary measurements run first, so that the GPU clocks have
    # long reached their loaded level when the headline steps are timed.
    c = setup_decode(args.workload, torch, sa, synth)
    w, sh, B, alg = c["w"], c["w"]["shape"], c["B"], c["alg"]
    others = [x for x in args.other_workloads.split(",") if x and x != "none" and x != args.workload]
    other_lines = {name: run_other_decode(args, torch, sa, synth, name) for name in others}
    prefill_lines = {}
    if not args.no_prefill:
        prefill_lines["prefill"] = run_prefill(args, torch, sa, synth)
        prefill_lines["prefill_varlen"] = run_prefill(args, torch, sa, synth, "prefill_varlen_8x4k")
    supp = supplementary_decode(args, torch, sa, synth, c)
    stages, ms_marked = time_stages(torch, sa, c, args.steps)
    log(f"steps with an event after every kernel: {ms_marked:.3f} ms/step; stages " +
        ", ".join(f"{k} {v * 1e3:.1f}us" for k, v in stages.items()))
    cold = time_flushed(torch, sa, c, args.flush_steps) if args.flush_steps > 0 else None

    # the headline: W warm-up steps, then exactly K plain steps between two synchronisations
    log(f"warmup {args.warmup} steps ({len(c['kernels'])} kernels per step: {', '.join(c['kernels'])})")
    ms = time_back_to_back(torch, c["plain"], args.steps, args.warmup)
    log(f"timed {args.steps} steps: {ms:.4f} ms/step")
    value = B / (ms / 1e3)
    t_idx = stages.get("indexer")
    roof = None
    if t_idx:
        achieved = alg["indexer_bytes"] / (t_idx / 1e3) / 1e9
        traffic = traffic_from_profiles(TRAFFIC_KERNEL + "/" + args.workload, 1)
        roof = {"bound": "hbm", "kernel": TRAFFIC_KERNEL, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "avg_ms": round(t_idx, 5), "algorithmic_bytes": alg["indexer_bytes"]}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "context": "uniform[16384,131072]" if
                   args.workload == "decode_b64_ctx16k_128k" else int(w["context_lens"].max()),
                   "topk": sh.topk, "heads": sh.num_heads, "qk_dim": sh.qk_dim, "v_dim": sh.v_dim,
                   "indexer": f"{sh.idx_heads}x{sh.idx_dim}", "block_size": sh.block_size, "out": "fp32",
                   "parallelism": "single GPU"},
        "hbm_gbps": round(alg["bytes"] / (ms / 1e3) / 1e9, 1),
        "hbm_frac": round(alg["bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": alg["bytes"],
        "stages_us": {k: round(v * 1e3, 2) for k, v in stages.items()},
        "ms_per_step_with_stage_events": round(ms_marked, 4),
        "cold_cache_ms_per_step": round(cold[0], 4) if cold else None,
        "roofline": roof,
    }
    t_att = stages.get("attention")
    if t_att:
        # the attention kernel against both of its bounds (its merge is a separate kernel)
        line["attention_roofline"] = {
            "kernel": "attend_kernel<576, 512, 2>", "avg_ms": round(t_att, 5),
            "hbm_gbps": round(alg["attention_bytes"] / (t_att / 1e3) / 1e9, 1),
            "hbm_frac": round(alg["attention_bytes"] / (t_att / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "mfma_tflops": round(alg["attention_flops"] / (t_att / 1e3) / 1e12, 1),
            "mfma_frac": round(alg["attention_flops"] / (t_att / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    if peaks:
        line["measured_peaks"] = peaks
    line.update(supp)
    line.update(prefill_lines)
    if other_lines:
        line["other_workloads"] = other_lines
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on up to {args.cpu_seconds:.0f}s of rows")
        line["cpu_baseline"] = cpu_baseline(args, w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
