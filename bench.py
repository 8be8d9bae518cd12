#!/usr/bin/env python3
"""Benchmark of the decode indexer (scoring + top-k) on one MI355X.

Workload: the fp8 decode batch -- 32 requests, seq_len ~ U[4096, 32768],
page 64, 20,000-page pool, H=64 index heads, head_dim 128, top-k 2048,
next_n=1 (synthetic, seeded).  A step is the whole decode path over the
batch: row expansion, page gather, bf16-MFMA scoring with the ReLU-weighted
head sum (idx_logits_paged), then the per-row top-k (idx_topk) -- the same
two launches idx_decode_topk makes, called separately so that HIP events
between them time the scorer on its own.

Timing: inputs are resident in HBM before the timed region.  The pool
(169 MB) would fit the 256 MiB MALL, so each step reads one of `--copies`
identical pools in rotation (8 x 169 MB by default); between two uses of a
pool ~550 MB of other keys stream through, so the keys come from HBM.  K
steps are bracketed by synchronisation (the value).  Then each kernel is
launched K times back to back (the scorer still on the rotated pools)
between HIP events on the launch stream; the mean interval per launch is the
launch duration used for the roofline.

Prints one JSON line.  `--summarize-prof DIR...` turns rocprofv3 outputs
(kernel-trace stats and FETCH_SIZE / WRITE_SIZE counter runs) into
profiles/score_kernel_fp8_decode_32req.{md,json}, which later runs use for
`traffic`.

`--prefill` measures the prefill path instead (a separate line, not the
benchmark's value): the chunks the planner makes for the prefill workload
(2 requests x 16384 queries over 65536 keys, H=64, D=128, top-k 2048), each
scored by idx_logits_paged on its rows and selected by idx_topk; the scorer
is reported against the bf16 dense MFMA peak.  `--summarize-prefill` turns
its rocprofv3 kernel-trace and SQ-counter runs into
profiles/score_block_kernel_fp8_prefill.md.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "index keys scored/sec + top-k rows/sec, 1×MI355X; % of HBM (decode) / MFMA (prefill) peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PREFILL_KERNEL_SUBSTR = "score_block_kernel<128, false, 2>"
PREFILL_PROFILE_NAME = "score_block_kernel_fp8_prefill"
PROFILE_NAME = "score_kernel_fp8_decode_32req"
KERNEL_SUBSTR = "score_kernel<128, false, 2>"   # scorer: D=128, fp8, 64 heads
TOPK_SUBSTR = "topk_kernel<"
CALIB_SUBSTR = "AUnaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float>"
CSRC = os.path.join(ROOT, "sparse_attention_indexer_decode_amd", "csrc")
DECODE_WORKLOADS = {
    "C1": "tiny fp8 decode: 1 request, L=300, 8-page pool, H=4, head_dim 32, top-k 64",
    "V4": "compressed fp8 decode: 64 requests x 131072 tokens, compress ratio 4 (32768 keys each), 256-token "
          "pages, H=64, head_dim 128, top-k 2048, fp8 e4m3 keys + fp32 scales",
    "C2": "fp8 decode batch: 32 requests, next_n=1, seq_len ~ U[4096, 32768], page 64, 20k-page pool, H=64, "
          "head_dim 128, top-k 2048, fp8 e4m3 keys + fp32 scales",
    "C3": "MTP decode: 128 requests, next_n=2 padded grid, decode_lens in {1, 2}, seq_len log-uniform in "
          "[512, 131072], page 64, H=64, head_dim 128, top-k 2048, fp8 e4m3 keys + fp32 scales",
    "C4": "MXFP4 long-context decode: 64 requests x 131072 keys, page 64, H=64, head_dim 128, top-k 2048, "
          "e2m1 keys + ue8m0 block scales",
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl) -> dict:
    """Bytes one scorer launch must move at minimum: every live key row once
    (D fp8 codes + 4-byte scale = 132 B at D=128), one fp32 logit written per
    key (4 B), each row's bf16 q and fp32 w, the block-table entries of the
    live pages and the lengths."""
    stored = wl.seq_lens.astype("int64") // wl.compress_ratio
    keys = int(stored.sum())
    rows = wl.num_req * wl.next_n
    pages = int(sum(-(-int(L) // wl.page_size) for L in stored))
    b = {
        "keys": keys * wl.row_bytes,
        "logits": keys * 4,
        "q": rows * wl.heads * wl.head_dim * 2,
        "w": rows * wl.heads * 4,
        "block_table": pages * 4,
        "lengths": wl.num_req * 4,
    }
    b["total"] = sum(b.values())
    return b


def scored_keys(wl) -> int:
    """Keys the fused decode scores: sum of L over grid rows with L > k
    (shorter rows are causal-filled without scoring)."""
    total = 0
    for b in range(wl.num_req):
        dl = wl.next_n if wl.decode_lens is None else int(wl.decode_lens[b])
        for i in range(min(dl, wl.next_n)):
            L = (int(wl.seq_lens[b]) - dl + i + 1) // wl.compress_ratio
            total += L if L > wl.topk else 0
    return total


def _oracle_cores() -> int:
    """Threads the oracle's numpy (BLAS) uses on this host."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(wl, budget_s: float = 10.0) -> dict:
    """The oracle (numpy, float64) on the host cores: whole requests of the
    batch in order, cycling over the batch, until about `budget_s` seconds
    of work are done."""
    import oracle

    threads = _oracle_cores()
    keys = 0
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < budget_s:
        b = done % wl.num_req
        lg = oracle.pipeline.decode_logits(wl, requests=[b])
        oracle.pipeline.decode_topk(wl, lg, requests=[b])
        keys += int(sum(len(v) for v in lg.values() if len(v) > wl.topk))
        done += 1
    dt = time.perf_counter() - t0
    return {"value": keys / dt, "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} requests of the {wl.num_req}-request batch in order, cycling "
                      f"({done / wl.num_req:.1f} passes, {keys} keys, {dt:.1f} s): dequantise, fp64 logits, "
                      f"top-k; cpus visible {len(os.sched_getaffinity(0))}"}


def load_traffic(per_launch_bytes: int):
    """The scorer's measured HBM bytes per launch from the committed counter
    profile, or None unless that profile was taken on the current kernel
    source and on this workload (the same algorithmic bytes per launch)."""
    path = os.path.join(ROOT, "profiles", PROFILE_NAME + ".json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        prof = json.load(f)
    if prof.get("source_hash") != kernel_source_hash():
        return None, prof
    if prof.get("algorithmic_bytes_per_launch") != per_launch_bytes:
        return None, prof
    t = prof.get("traffic_bytes_per_launch")
    return t, prof


def run(args):
    import numpy as np
    import torch

    import sparse_attention_indexer_decode_amd as idx
    from workloads import config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = config(args.config)
    pools = [torch.from_numpy(wl.cache).to(dev)]
    for _ in range(args.copies - 1):
        pools.append(pools[0].clone())
    caches = [idx.Cache(p, wl.head_dim, wl.fmt, wl.page_size) for p in pools]
    bt = torch.from_numpy(wl.block_table).to(dev)
    seq = torch.from_numpy(wl.seq_lens).to(dev)
    dl = None if wl.decode_lens is None else torch.from_numpy(wl.decode_lens).to(dev)
    rows = idx.Rows.decode(bt, seq, int(wl.seq_lens.max()), next_n=wl.next_n, decode_lens=dl,
                           compress_ratio=wl.compress_ratio)
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wl.w).to(dev)
    k = wl.topk
    R = rows.num_rows
    outs = torch.empty((R, k), dtype=torch.int32, device=dev)
    ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_DECODE_TOPK, caches[0], rows, wl.heads, k), dev)
    ML = int(wl.seq_lens.max()) // wl.compress_ratio   # keys of the longest row
    stride = -(-ML // 64) * 64
    logits = torch.empty((R, stride), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        idx.idx_logits_paged(caches[i % len(caches)], rows, q, w, logits, ws, stream)
        if ev is not None:
            ev[1].record(stream)
        idx.idx_topk(logits, rows, k, outs, ws, stream)
        if ev is not None:
            ev[2].record(stream)

    if args.calib:
        # a plain elementwise copy of known size (reads and writes calib_mib
        # MiB), for scaling the FETCH/WRITE counters
        src = torch.ones((args.calib_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    first = outs.clone()
    # the public one-call entry point makes the same two launches
    fused = torch.full_like(outs, -7)
    idx.idx_decode_topk(caches[0], rows, q, w, k, fused, ws, stream)
    torch.cuda.synchronize()
    assert torch.equal(first, fused), "idx_decode_topk differs from idx_logits_paged + idx_topk"

    # timed region: K whole steps back to back (wall clock between syncs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert torch.equal(first, outs), "decode top-k is not deterministic across steps"
    # per-kernel launch durations for the roofline: HIP events on the launch
    # stream around K back-to-back launches of one kernel (the scorer on the
    # rotated pools, the selector on the step's logits), divided by K, in
    # chunks so that min and spread are visible
    def timed(fn, n, chunk=20):
        per = []
        for c0 in range(0, n, chunk):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            m = min(chunk, n - c0)
            e0.record(stream)
            for i in range(m):
                fn(c0 + i)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / m)
        return per

    torch.cuda.synchronize()
    score_ms = timed(lambda i: idx.idx_logits_paged(caches[(args.warmup + i) % len(caches)], rows, q, w, logits, ws,
                                                    stream), args.steps)
    topk_ms = timed(lambda i: idx.idx_topk(logits, rows, k, outs, ws, stream), args.steps)
    torch.cuda.synchronize()
    assert torch.equal(first, outs), "decode top-k is not deterministic across steps"

    # warm-MALL reference: the same pool back to back (context only)
    for _ in range(5):
        step(0)
    ws_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ws_ev[0].record(stream)
    for _ in range(20):
        step(0)
    ws_ev[1].record(stream)
    torch.cuda.synchronize()
    warm_ms = ws_ev[0].elapsed_time(ws_ev[1]) / 20

    keys_scored = scored_keys(wl)
    ms_per_step = wall * 1000.0 / args.steps
    score_avg_ms = float(np.mean(score_ms))
    ab = algorithmic_bytes(wl)
    achieved = ab["total"] / (score_avg_ms * 1e-3) / 1e9
    traffic, prof = load_traffic(ab["total"])
    res = {
        "metric": METRIC,
        "value": keys_scored / (ms_per_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DECODE_WORKLOADS[wl.name],
                   "name": wl.name, "requests": wl.num_req, "rows": R, "keys_scored": keys_scored,
                   "cache_fmt": "mxfp4" if wl.fmt == "mxfp4" else "fp8_e4m3", "pool_copies_rotated": args.copies},
        "rows_per_s": R / (ms_per_step * 1e-3),
        "scorer_ms_avg": score_avg_ms,
        "scorer_ms_min": float(np.min(score_ms)),
        "topk_ms_avg": float(np.mean(topk_ms)),
        "warm_mall_ms_per_step": warm_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": ab["total"],
                     "kernel": f"score_kernel<D={wl.head_dim}, {wl.fmt}, {wl.heads} heads> (idx_logits_paged)"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(res), flush=True)


def run_prefill(args):
    """The prefill workload's planner chunks: per chunk one scorer and one
    selector launch over all of its rows."""
    import numpy as np
    import torch

    import sparse_attention_indexer_decode_amd as idx
    from workloads import config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = config("C5")
    cache = idx.Cache(torch.from_numpy(wl.cache).to(dev), wl.head_dim, wl.fmt)
    bt = torch.from_numpy(wl.block_table).to(dev)
    seq = torch.from_numpy(wl.seq_lens).to(dev)
    qsl = torch.from_numpy(np.concatenate([[0], np.cumsum(wl.query_lens)]).astype(np.int32)).to(dev)
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wl.w).to(dev)
    k = wl.topk
    recs = idx.idx_prefill_chunks(wl.seq_lens, wl.query_lens, 65536, 512 << 20)
    chunks = []
    flops = 0
    n_rows = 0
    for rec in recs:
        b0, b1 = rec["req_begin"], rec["req_end"]
        rows = idx.Rows.prefill(bt[b0:b1], seq[b0:b1], qsl[b0:b1 + 1], rec["q_begin"], rec["q_end"],
                                int(wl.seq_lens[b0:b1].max()))
        M, N = rec["q_end"] - rec["q_begin"], rec["total_seq_lens"]
        chunks.append((rows, q[rec["token_begin"]:rec["token_end"]], w[rec["token_begin"]:rec["token_end"]], M, N))
        # keys per row: L = seq_len - query_len + j + 1 for query j of its request
        for b in range(b0, b1):
            qs = int(wl.query_lens[b])
            j = np.arange(qs)
            lo = max(0, rec["q_begin"] - int(np.sum(wl.query_lens[b0:b])))
            hi = min(qs, rec["q_end"] - int(np.sum(wl.query_lens[b0:b])))
            L = int(wl.seq_lens[b]) - qs + j[lo:hi] + 1
            flops += int(L.sum()) * 2 * wl.heads * wl.head_dim
            n_rows += max(0, hi - lo)
    big = max(M * N for _, _, _, M, N in chunks)
    logits_buf = torch.empty(big, dtype=torch.float32, device=dev)
    outs = torch.empty((max(c[3] for c in chunks), k), dtype=torch.int32, device=dev)
    ws_bytes = max(max(idx.idx_workspace_bytes(idx.IDX_OP_LOGITS, cache, c[0], wl.heads, 0),
                       idx.idx_workspace_bytes(idx.IDX_OP_TOPK, None, c[0], 0, k)) for c in chunks)
    ws = idx.new_workspace(ws_bytes, dev)
    stream = torch.cuda.current_stream()

    def one_pass(ev=None):
        for ci, (rows, qq, ww, M, N) in enumerate(chunks):
            lg = logits_buf[: M * N].view(M, N)
            if ev is not None:
                ev[ci][0].record(stream)
            idx.idx_logits_paged(cache, rows, qq, ww, lg, ws, stream)
            if ev is not None:
                ev[ci][1].record(stream)
            idx.idx_topk(lg, rows, k, outs[:M], ws, stream)
            if ev is not None:
                ev[ci][2].record(stream)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_pass()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in chunks]
    one_pass(evs)
    torch.cuda.synchronize()
    score_ms = sum(e[0].elapsed_time(e[1]) for e in evs)
    topk_ms = sum(e[1].elapsed_time(e[2]) for e in evs)
    tflops = flops / (score_ms * 1e-3) / 1e12
    res = {
        "metric": "prefill indexer: query rows scored and selected per second, 1xMI355X",
        "value": n_rows / wall, "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill: 2 requests x 16384 queries, seq_len 65536, H=64, head_dim 128, "
                               "top-k 2048, fp8 keys; planner chunks of <= 65536 keys and <= 512 MiB of logits",
                   "name": wl.name, "chunks": len(chunks), "rows": n_rows},
        "scorer_ms_per_pass": score_ms, "topk_ms_per_pass": topk_ms,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_PEAK_TFLOPS, "traffic": None, "algorithmic_flops_per_pass": flops,
                     "kernel": "score_block_kernel<D=128, fp8, 64 heads> (idx_logits_paged on prefill rows)"},
    }
    print(json.dumps(res), flush=True)


def run_cache_write(args):
    """The index-cache write: 64 x 131072 = 8,388,608 new bf16 key tokens
    quantised into a pool of exactly that many slots (pages in random order,
    tokens in order within a page), fp8 and MXFP4, one launch each; a
    separate line per format."""
    import numpy as np
    import torch

    import sparse_attention_indexer_decode_amd as idx

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    T, D = 64 * 131072, 128
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    k = torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16)
    # 64 requests of 131072 tokens: each request's pages dealt from one
    # random permutation of the pool, tokens in order within a page
    pages = torch.randperm(T // 64, generator=g, device=dev)
    t = torch.arange(T, device=dev)
    slots = pages[t // 64] * 64 + t % 64
    ws = idx.new_workspace(256, dev)
    stream = torch.cuda.current_stream()
    for fmt in ("fp8", "mxfp4"):
        rb = D + 4 if fmt == "fp8" else D // 2 + D // 32
        page_bytes = (64 * rb + 15) // 16 * 16
        pool = torch.zeros((T // 64, page_bytes), dtype=torch.uint8, device=dev)
        cache = idx.Cache(pool, D, fmt)
        for _ in range(args.warmup):
            idx.idx_cache_write(cache, k, slots, ws, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            idx.idx_cache_write(cache, k, slots, ws, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        alg = T * (2 * D + rb + 8)          # bf16 key read, row written, int64 slot read
        gbs = alg / (ms * 1e-3) / 1e9
        res = {
            "metric": "index-cache write: key tokens quantised and stored per second, 1xMI355X",
            "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"cache write: {T} bf16 key tokens, head_dim {D}, {fmt} rows of {rb} B, "
                                   "int64 slots of 64-token pages dealt at random from a pool of exactly that many slots",
                       "fmt": fmt, "tokens": T},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_launch": alg,
                         "kernel": f"cache_write_kernel<D={D}, {fmt}> (idx_cache_write)"},
        }
        if not args.no_cpu_baseline:
            import oracle
            sample = 32768
            kb = k[:sample].view(torch.int16).cpu().numpy().view(np.uint16)
            t0 = time.perf_counter()
            n = 0
            while time.perf_counter() - t0 < args.cpu_budget / 4:
                oracle.cache_write.quantize_rows(kb, fmt)
                n += sample
            dt = time.perf_counter() - t0
            res["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s", "cores": _oracle_cores(), "kind": "oracle",
                                   "sample": f"the first {sample} tokens quantised repeatedly ({n} tokens, {dt:.1f} s)"}
        print(json.dumps(res), flush=True)
        del pool


def summarize_prefill(stats_dir, pmc_dir, commands, bench_json):
    """Kernel time and SQ counters of the prefill scorer ->
    profiles/score_block_kernel_fp8_prefill.md"""
    import numpy as np

    stats = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    lines = []
    for r in _csv_rows(stats[0]):
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    for r in _csv_rows(files[0]):
        if PREFILL_KERNEL_SUBSTR not in r.get("Kernel_Name", ""):
            continue
        per.setdefault(r["Dispatch_Id"], {}).setdefault(r["Counter_Name"], 0.0)
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
    names = sorted({c for d in per.values() for c in d})
    med = {c: float(np.median([d[c] for d in per.values() if c in d])) for c in names}
    with open(bench_json) as f:
        bl = json.loads(f.read().strip().splitlines()[-1])
    md = ["# Prefill scorer on the prefill workload (2 x 16384 queries over 65536 keys, H=64, D=128)", "",
          "Commands (run from the repository root on one MI355X):", ""]
    md += [f"    {c}" for c in commands]
    md += ["", "## rocprofv3 --kernel-trace --stats", "",
           "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"] + lines
    md += ["", "## bench.py --prefill", "",
           f"- scorer {bl['scorer_ms_per_pass']:.2f} ms per pass of {bl['config']['chunks']} chunks (HIP events) = "
           f"{bl['roofline']['achieved']:.0f} TFLOP/s of algorithmic bf16 work = "
           f"{bl['roofline']['frac'] * 100:.1f} % of the 2.5 PFLOP/s dense bf16 peak",
           f"- selector {bl['topk_ms_per_pass']:.2f} ms per pass; {bl['value']:.4g} rows/s end to end",
           "", "## SQ counters of one scorer dispatch (rocprofv3 --pmc, summed over the chip; median over dispatches)",
           ""] + [f"- {c}: {med[c]:.4g}" for c in names]
    md += [f"", f"- kernel source hash {kernel_source_hash()}"]
    with open(os.path.join(ROOT, "profiles", PREFILL_PROFILE_NAME + ".md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


# ---------------------------------------------------------------------------
# rocprofv3 output -> profiles/
# ---------------------------------------------------------------------------

def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize(dirs, commands, bench_json=None):
    """dirs: rocprofv3 output dirs of (1) --kernel-trace --stats, (2) --pmc
    FETCH_SIZE, (3) --pmc WRITE_SIZE runs of this script."""
    import numpy as np

    from workloads import config

    out = {"source_hash": kernel_source_hash(), "commands": commands}
    stats = glob.glob(os.path.join(dirs[0], "**", "*kernel_stats.csv"), recursive=True)
    rows = _csv_rows(stats[0])
    lines = []
    for r in rows:
        if KERNEL_SUBSTR in r["Name"]:
            out["kernel"] = r["Name"]
            out["calls"] = int(r["Calls"])
            out["avg_ns"] = float(r["AverageNs"])
            out["min_ns"] = float(r["MinNs"])
            out["max_ns"] = float(r["MaxNs"])
        if TOPK_SUBSTR in r["Name"]:
            out["topk_kernel"] = r["Name"]
            out["topk_avg_ns"] = float(r["AverageNs"])
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")

    def counter(d, cname):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        per_kernel, copy_vals = [], []
        for r in _csv_rows(files[0]):
            if r.get("Counter_Name") != cname:
                continue
            v = float(r["Counter_Value"])
            name = r.get("Kernel_Name", "")
            if KERNEL_SUBSTR in name:
                per_kernel.append(v)
            elif CALIB_SUBSTR in name:
                copy_vals.append(v)
        return per_kernel, copy_vals

    bl = None
    if bench_json:
        with open(bench_json) as f:
            bl = json.loads(f.read().strip().splitlines()[-1])
        out["bench_scorer_ms_avg"] = bl["scorer_ms_avg"]
        out["bench_topk_ms_avg"] = bl["topk_ms_avg"]
    wl = config("C2")
    ab = algorithmic_bytes(wl)
    fetch, fcopy = counter(dirs[1], "FETCH_SIZE")
    write, wcopy = counter(dirs[2], "WRITE_SIZE")
    calib_bytes = 256 << 20
    # counters are in KiB per dispatch; scale by what they read for a copy of known size
    f_scale = calib_bytes / (np.median(fcopy) * 1024) if fcopy else 1.0
    w_scale = calib_bytes / (np.median(wcopy) * 1024) if wcopy else 1.0
    out["fetch_kib_per_launch"] = float(np.median(fetch)) if fetch else None
    out["write_kib_per_launch"] = float(np.median(write)) if write else None
    out["copy_fetch_kib"] = float(np.median(fcopy)) if fcopy else None
    out["copy_write_kib"] = float(np.median(wcopy)) if wcopy else None
    out["fetch_scale"] = f_scale
    out["write_scale"] = w_scale
    if fetch and write:
        out["traffic_bytes_per_launch"] = (out["fetch_kib_per_launch"] * f_scale
                                           + out["write_kib_per_launch"] * w_scale) * 1024
    out["algorithmic_bytes_per_launch"] = ab["total"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", PROFILE_NAME + ".json"), "w") as f:
        json.dump(out, f, indent=1)
    md = [f"# Scorer kernel on the fp8 decode batch (32 x U[4096, 32768], H=64, D=128, k=2048)", "",
          "Commands (run from the repository root on one MI355X):", ""]
    md += [f"    {c}" for c in commands]
    md += ["", "## rocprofv3 --kernel-trace --stats", "",
           "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"] + lines
    if bl is not None:
        md += ["", "## HIP-event launch durations in the same benchmark (bench.py: 200 back-to-back launches of each "
               "kernel between events, mean per launch)", "",
               f"- scorer {bl['scorer_ms_avg'] * 1e3:.2f} us per launch (rocprofv3 kernel time "
               f"{out.get('avg_ns', float('nan')) / 1e3:.2f} us; the events also hold the gap between launches)",
               f"- selector {bl['topk_ms_avg'] * 1e3:.2f} us per launch (rocprofv3 "
               f"{out.get('topk_avg_ns', float('nan')) / 1e3:.2f} us)",
               f"- step {bl['ms_per_step'] * 1e3:.2f} us wall clock; {bl['value']:.4g} keys/s; scorer "
               f"{bl['roofline']['achieved']:.0f} GB/s algorithmic = {bl['roofline']['frac'] * 100:.1f} % of 8 TB/s"]
    md += ["", "## HBM traffic of the scorer kernel (rocprofv3 --pmc, per dispatch)", "",
           f"- FETCH_SIZE {out['fetch_kib_per_launch']} KiB, WRITE_SIZE {out['write_kib_per_launch']} KiB",
           f"- plain 256 MiB copy reads as FETCH {out['copy_fetch_kib']} KiB / WRITE {out['copy_write_kib']} KiB "
           f"-> scale {f_scale:.4f} / {w_scale:.4f}",
           f"- traffic per launch {out.get('traffic_bytes_per_launch')} B vs algorithmic {ab['total']} B",
           f"- kernel source hash {out['source_hash']}"]
    with open(os.path.join(ROOT, "profiles", PROFILE_NAME + ".md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calib", action="store_true", help="also run a plain copy for counter scaling")
    ap.add_argument("--calib-mib", type=int, default=256)
    ap.add_argument("--summarize-prof", nargs=3, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--commands", nargs="*", default=[])
    ap.add_argument("--bench-json", default=None)
    ap.add_argument("--prefill", action="store_true", help="measure the prefill path instead (separate line)")
    ap.add_argument("--summarize-prefill", nargs=2, metavar=("STATS_DIR", "PMC_DIR"))
    ap.add_argument("--cache-write", action="store_true", help="measure the index-cache write instead (separate lines)")
    args = ap.parse_args()
    if args.summarize_prof:
        summarize(args.summarize_prof, args.commands, args.bench_json)
        return
    if args.summarize_prefill:
        summarize_prefill(args.summarize_prefill[0], args.summarize_prefill[1], args.commands, args.bench_json)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; --gpus must be 1 (multi-GPU sharding is "
                                   "described, not implemented)"}), flush=True)
        sys.exit(2)
    if args.prefill:
        run_prefill(args)
        return
    if args.cache_write:
        run_cache_write(args)
        return
    run(args)


if __name__ == "__main__":
    main()
