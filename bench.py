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
on the library's stream between its kernels inside the timed region.
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
    # the indexer kernel alone: key rows + score writes + per-row query/weights + block table
    idx_bytes = int((ctx * (sh.idx_dim * 2 + 4)).sum() + len(ctx) * sh.idx_heads * (2 * sh.idx_dim + 4) +
                    (4 * blocks).sum())
    return dict(bytes=total, scan=scan, gather=gather, flops=flops, indexer_bytes=idx_bytes)


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


def run_decode(args, torch, sa, synth):
    spec = synth.WORKLOADS[args.workload]
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
    call = lambda ev: sa.sparse_attn_decode_profiled(p, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"], ev,
                                                     workspace=ws, outputs=outs)
    n_marks = call([])[3]
    kernels = ["indexer", "topk", "attention", "merge"][:n_marks - 1] if max_ctx > p.topk else \
        ["topk", "attention", "merge"][:n_marks - 1]
    plain = lambda: sa.sparse_attn_decode(p, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"], workspace=ws,
                                          outputs=outs)
    log(f"warmup {args.warmup} steps ({n_marks - 1} kernels per step: {', '.join(kernels)})")
    for _ in range(args.warmup):
        plain()
    torch.cuda.synchronize()
    # The timed steps are plain calls: an event recorded between two kernels
    # holds the next one back, so per-stage times come from separate steps.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plain()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    # The same step with each sequence's current token appended to the cache
    # first (sparse_attn_decode_append; the same token every step, so the cache
    # holds the same values throughout), timed like the plain step right after it.
    append_ms = None
    if args.append_steps > 0:
        nk_np, ni_np = synth.new_tokens(w)
        nk = torch.from_numpy(nk_np).view(torch.bfloat16).cuda()
        ni = torch.from_numpy(ni_np).view(torch.bfloat16).cuda()
        app = lambda: sa.sparse_attn_decode_append(p, d["cache"], max_ctx, nk, ni, d["q"], d["idx_q"], d["idx_w"],
                                                   workspace=ws, outputs=outs)
        for _ in range(args.warmup):
            app()
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for _ in range(args.append_steps):
            app()
        torch.cuda.synchronize()
        append_ms = (time.perf_counter() - ta) * 1e3 / args.append_steps
        tb = time.perf_counter()
        for _ in range(args.steps):
            plain()
        torch.cuda.synchronize()
        again = (time.perf_counter() - tb) * 1e3 / args.steps
        log(f"decode with append: {append_ms:.3f} ms/step (plain step again after it: {again:.3f} ms)")
    # Run-time tuning of the attention split count on this batch, then the
    # configured call timed like the plain one.
    tuned = None
    if args.tune:
        splits, tune_us = sa.decode_tune(p, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"], reps=10)
        wst = torch.empty(sa.decode_workspace_size_cfg(p, B, max_ctx, splits), dtype=torch.uint8, device="cuda")
        cfg = lambda: sa.sparse_attn_decode_cfg(p, d["cache"], max_ctx, splits, d["q"], d["idx_q"], d["idx_w"],
                                                workspace=wst, outputs=outs)
        for _ in range(args.warmup):
            cfg()
        torch.cuda.synchronize()
        tc = time.perf_counter()
        for _ in range(args.steps):
            cfg()
        torch.cuda.synchronize()
        tuned = dict(attn_splits=splits, ms=(time.perf_counter() - tc) * 1e3 / args.steps, tune_us=tune_us)
        log(f"tuned: {splits} attention splits per row, {tuned['ms']:.3f} ms/step (tuner's own mean {tune_us:.1f} us)")
        del wst
    # Block-granular selection over the same batch: k / block_size whole cache
    # blocks per row (the same number of attended token slots), timed the same way.
    blocks_ms = None
    if args.blocks_steps > 0:
        from dataclasses import replace
        sh = w["shape"]
        pb = sa.Params.from_shape(replace(sh, topk=sh.topk // sh.block_size))
        wsb = torch.empty(sa.decode_blocks_workspace_size(pb, B, max_ctx), dtype=torch.uint8, device="cuda")
        outb = sa._outputs(pb, B, "cuda", True)
        blk = lambda: sa.sparse_attn_decode_blocks(pb, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"],
                                                   workspace=wsb, outputs=outb)
        for _ in range(args.warmup):
            blk()
        torch.cuda.synchronize()
        tb = time.perf_counter()
        for _ in range(args.blocks_steps):
            blk()
        torch.cuda.synchronize()
        blocks_ms = (time.perf_counter() - tb) * 1e3 / args.blocks_steps
        log(f"decode with block selection ({pb.topk} blocks of {sh.block_size}): {blocks_ms:.3f} ms/step")
        del wsb, outb
    events = [[sa.HipEvent() for _ in range(n_marks)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for s in range(args.steps):
        call(events[s])
    torch.cuda.synchronize()
    ms_marked = (time.perf_counter() - t2) * 1e3 / args.steps
    log(f"steps with an event after every kernel: {ms_marked:.3f} ms/step")
    per_kernel = {k: [] for k in kernels}
    for ev in events:
        for i, k in enumerate(kernels):
            per_kernel[k].append(ev[i].elapsed_ms(ev[i + 1]))
    stages = {k: statistics.mean(v) for k, v in per_kernel.items()}
    log(f"timed {args.steps} steps: {ms:.3f} ms/step; stages " +
        ", ".join(f"{k} {v * 1e3:.1f}us" for k, v in stages.items()))

    # the same step with a 1 GiB write between steps (HBM-cold caches), events only
    cold = []
    if args.flush_steps > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        for _ in range(args.flush_steps):
            flush.fill_(1.0)
            ev = [sa.HipEvent() for _ in range(n_marks)]
            call(ev)
            torch.cuda.synchronize()
            cold.append(ev[0].elapsed_ms(ev[-1]))
        del flush
    alg = decode_algorithmic(w)
    return w, dict(ms=ms, stages=stages, cold_ms=statistics.median(cold) if cold else None, alg=alg,
                   per_kernel=per_kernel, append_ms=append_ms, ms_marked=ms_marked, blocks_ms=blocks_ms,
                   tuned=tuned)


def run_other_decodes(args, torch, sa, synth, names):
    """The other decode configurations, timed like the main one (fewer steps, no flush)."""
    res = {}
    for name in names:
        sub = argparse.Namespace(**vars(args))
        sub.workload, sub.steps, sub.warmup, sub.flush_steps, sub.append_steps = name, 20, 20, 0, 0
        sub.blocks_steps = 0
        w, dec = run_decode(sub, torch, sa, synth)
        B = len(w["context_lens"])
        res[name] = {"ms_per_step": round(dec["ms"], 4), "tokens_per_s": round(B / (dec["ms"] / 1e3), 1),
                     "hbm_gbps": round(dec["alg"]["bytes"] / (dec["ms"] / 1e3) / 1e9, 1),
                     "hbm_frac": round(dec["alg"]["bytes"] / (dec["ms"] / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "algorithmic_bytes_per_step": dec["alg"]["bytes"],
                     "stages_us": {k: round(v * 1e3, 2) for k, v in dec["stages"].items()}}
        if dec["tuned"]:
            res[name]["tuned"] = {"attn_splits": dec["tuned"]["attn_splits"],
                                  "ms_per_step": round(dec["tuned"]["ms"], 4),
                                  "tokens_per_s": round(B / (dec["tuned"]["ms"] / 1e3), 1)}
        del w, dec
        torch.cuda.empty_cache()
    return res


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
    log(f"{spec.name}: {ms:.2f} ms/step, stages {res['stages_ms']}")
    return res


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
    ap.add_argument("--flush-steps", type=int, default=5, help="extra steps timed after a 1 GiB cache flush")
    ap.add_argument("--prefill-steps", type=int, default=2)
    ap.add_argument("--append-steps", type=int, default=20,
                    help="steps of the decode call that also appends each sequence's current token to the "
                         "cache (sparse_attn_decode_append), timed like the plain steps right after them")
    ap.add_argument("--blocks-steps", type=int, default=20,
                    help="steps of block-granular decode (sparse_attn_decode_blocks, k / block_size blocks per "
                         "row) over the same batch")
    ap.add_argument("--no-tune", dest="tune", action="store_false",
                    help="skip the run-time tuning of the attention split count (sa_decode_tune)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--other-workloads", default="none",
                    help="comma-separated decode workloads also timed, e.g. decode_b32_ctx8k,decode_b4_ctx1m "
                         "(supplementary, not the metric; off by default so that kernel traces of the default "
                         "command hold the headline workload only)")
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

    w, dec = run_decode(args, torch, sa, synth)
    sh = w["shape"]
    B = len(w["context_lens"])
    value = B / (dec["ms"] / 1e3)
    alg = dec["alg"]
    t_idx = dec["stages"].get("indexer")
    roof = None
    if t_idx:
        achieved = alg["indexer_bytes"] / (t_idx / 1e3) / 1e9
        traffic = traffic_from_profiles(TRAFFIC_KERNEL + "/" + args.workload, 1)
        roof = {"bound": "hbm", "kernel": TRAFFIC_KERNEL, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "avg_ms": round(t_idx, 5)}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dec["ms"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "context": "uniform[16384,131072]" if
                   args.workload == "decode_b64_ctx16k_128k" else int(w["context_lens"].max()),
                   "topk": sh.topk, "heads": sh.num_heads, "qk_dim": sh.qk_dim, "v_dim": sh.v_dim,
                   "indexer": f"{sh.idx_heads}x{sh.idx_dim}", "block_size": sh.block_size, "out": "fp32",
                   "parallelism": "single GPU"},
        "hbm_gbps": round(alg["bytes"] / (dec["ms"] / 1e3) / 1e9, 1),
        "hbm_frac": round(alg["bytes"] / (dec["ms"] / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": alg["bytes"],
        "stages_us": {k: round(v * 1e3, 2) for k, v in dec["stages"].items()},
        "ms_per_step_with_stage_events": round(dec["ms_marked"], 4),
        "cold_cache_ms_per_step": round(dec["cold_ms"], 4) if dec["cold_ms"] else None,
        "roofline": roof,
    }
    if dec.get("append_ms"):
        # supplementary: the same step appending each sequence's current token first
        line["decode_append"] = {"ms_per_step": round(dec["append_ms"], 4),
                                 "tokens_per_s": round(B / (dec["append_ms"] / 1e3), 1),
                                 "added_us": round((dec["append_ms"] - dec["ms"]) * 1e3, 2)}
    if dec.get("tuned"):
        # supplementary: the split count picked by sa_decode_tune on this batch
        t = dec["tuned"]
        line["decode_tuned"] = {"attn_splits": t["attn_splits"], "ms_per_step": round(t["ms"], 4),
                                "tokens_per_s": round(B / (t["ms"] / 1e3), 1)}
    if dec.get("blocks_ms"):
        # supplementary: block-granular selection over the same batch
        line["decode_blocks"] = {"ms_per_step": round(dec["blocks_ms"], 4),
                                 "tokens_per_s": round(B / (dec["blocks_ms"] / 1e3), 1),
                                 "kept_blocks": sh.topk // sh.block_size, "block_size": sh.block_size}
    if not args.no_prefill:
        line["prefill"] = run_prefill(args, torch, sa, synth)
        line["prefill_varlen"] = run_prefill(args, torch, sa, synth, "prefill_varlen_8x4k")
    others = [x for x in args.other_workloads.split(",") if x and x != "none" and x != args.workload]
    if others:
        line["other_workloads"] = run_other_decodes(args, torch, sa, synth, others)
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on up to {args.cpu_seconds:.0f}s of rows")
        line["cpu_baseline"] = cpu_baseline(args, w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
