#!/usr/bin/env python3
"""Benchmark of the indexer hot path (paged scoring + top-k) on one MI355X.

One run times all five synthetic workloads, each a full pass of the path
over one batch with its inputs already resident in HBM:

  C1 tiny fp8 decode      1 request, L=300, H=4, D=32, k=64
  C2 fp8 decode batch     32 requests, L ~ U[4096, 32768], H=64, D=128, k=2048
  C3 MTP decode           128 requests, next_n=2 padded grid, L log-uniform
                          [512, 131072], H=64, D=128, k=2048
  C4 MXFP4 decode         64 requests x 131072 keys, H=64, D=128, k=2048
  C5 chunked prefill      2 requests x 16384 queries over 65536 keys, the
                          planner's 16 chunks of <= 65536 keys and <= 512 MiB
                          of logits, H=64, D=128, k=2048

A decode step is idx_decode_topk on the batch (scorer launch + selector
launch); a prefill step is one pass over the planner's chunks, each scored
by idx_logits_paged and selected by idx_topk.  The headline line is the
largest workload, C5; every workload's numbers are under "configs".

Per workload:
  * value: keys scored per second (the sum over rows of L with L > k:
    causal-fill rows select without scoring) and rows per second, from K
    eager steps bracketed by synchronisation (wall clock), and again from a
    HIP graph of the same launches replayed K times;
  * roofline of the dominant kernel: its algorithmic bytes (decode: every
    live key row once, each real row's bf16 q and fp32 w, the block-table
    entries and lengths) or flops (prefill: 2 H D per (row, key) pair) per
    launch over its mean launch duration, HIP events on the launch stream
    around back-to-back launches; decode against 8 TB/s, prefill against the
    5.0 PFLOP/s dense fp8 MFMA peak the method sets as its bar (the kernel
    runs bf16 MFMA, whose dense peak, 2.5 PFLOP/s, is reported beside it);
  * whole_step: the same algorithmic work plus the top-k output over the
    whole step's wall time;
  * traffic: HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary for that kernel and workload,
    when it was taken on the current kernel source (else null);
  * cpu_baseline: the oracle (numpy float64) on the host cores, a bounded
    sample of the same workload.

Decode pools that would fit the 256 MiB MALL are read from `--copies`
rotated copies so that keys come from HBM.

`--summarize NAME STATS_DIR FETCH_DIR WRITE_DIR` turns rocprofv3 outputs of
a one-workload run (`--configs X`) into profiles/NAME.{md,json}.
`--cache-write` measures the index-cache write instead (separate lines);
`--configs V4` the compressed-cache decode.
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
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
CALIB_SUBSTR = "MulFunctor<float>"
CSRC = os.path.join(ROOT, "sparse_attention_indexer_decode_amd", "csrc")
ALL_CONFIGS = ("C1", "C2", "C3", "C4", "C5", "P2")
# pool-level workloads: (decode batch, pool size, pools kept, first kept, last kept)
POOL_WORKLOADS = {"P2": ("C2", 64, 32, 1, 2)}
WORKLOADS = {
    "C1": "tiny fp8 decode: 1 request, L=300, page 64, 8-page pool (random permutation), H=4, head_dim 32, "
          "top-k 64, next_n=1",
    "C2": "fp8 decode batch: 32 requests, next_n=1, seq_len ~ U[4096, 32768], page 64, 20k-page pool, H=64, "
          "head_dim 128, top-k 2048, fp8 e4m3 keys + fp32 scales",
    "C3": "MTP decode: 128 requests, next_n=2 padded grid, decode_lens in {1, 2}, seq_len log-uniform in "
          "[512, 131072], page 64, H=64, head_dim 128, top-k 2048, fp8 e4m3 keys + fp32 scales",
    "C4": "MXFP4 long-context decode: 64 requests x 131072 keys, page 64, H=64, head_dim 128, top-k 2048, "
          "e2m1 keys + ue8m0 block scales",
    "C5": "chunked prefill: 2 requests x 16384 queries, seq_len 65536, H=64, head_dim 128, top-k 2048, fp8 "
          "e4m3 keys + fp32 scales, page 64; planner chunks of <= 65536 keys and <= 512 MiB of logits (16 chunks)",
    "V4": "compressed fp8 decode: 64 requests x 131072 tokens, compress ratio 4 (32768 keys each), 256-token "
          "pages, H=64, head_dim 128, top-k 2048, fp8 e4m3 keys + fp32 scales",
    "P2": "pool-level decode: the fp8 decode batch (32 requests, seq_len ~ U[4096, 32768], H=64, head_dim 128), "
          "pools of 64 keys, 32 pools kept per row of which the first and the last two always",
}
# default rotated pool copies: enough that a pool is out of the MALL when it is read again
DEFAULT_COPIES = {"C1": 1, "C2": 8, "C3": 2, "C4": 2, "V4": 2, "P2": 8}
CPU_BUDGET_S = {"C1": 2.0, "C2": 5.0, "C3": 6.0, "C4": 6.0, "C5": 8.0, "V4": 5.0, "P2": 4.0}
PREFILL_WORKSPACE_TOKENS = 65536
PREFILL_LOGITS_BYTES = 512 << 20


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def scorer_kernel_name(wl) -> str:
    """The dominant kernel's name as rocprofv3 prints it (decode: the last
    template argument is the wave-pair form used for next_n = 2)."""
    mt = 2 if wl.heads > 32 else 1
    mx = "true" if wl.fmt == "mxfp4" else "false"
    if wl.kind == "prefill":
        return f"score_block_kernel<{wl.head_dim}, {mx}, {mt}>"
    pairs = "true" if wl.next_n == 2 else "false"
    return f"score_kernel<{wl.head_dim}, {mx}, {mt}, {pairs}>"


# ---------------------------------------------------------------------------
# Algorithmic work
# ---------------------------------------------------------------------------

def decode_rows(wl):
    """(key count L per real grid row, number of real rows)."""
    import numpy as np
    L = []
    for b in range(wl.num_req):
        dl = wl.next_n if wl.decode_lens is None else int(wl.decode_lens[b])
        for i in range(min(dl, wl.next_n)):
            L.append(max(0, int(wl.seq_lens[b]) - dl + i + 1) // wl.compress_ratio)
    return np.asarray(L, dtype=np.int64), len(L)


def decode_bytes(wl) -> dict:
    """Bytes a decode step must move at minimum: every live key row once per
    request (its rows share it), each real row's bf16 q and fp32 w, the
    block-table entries of the live pages and the lengths; the step adds the
    top-k output (k int32 per grid row)."""
    stored = wl.seq_lens.astype("int64") // wl.compress_ratio
    _, real = decode_rows(wl)
    pages = int(sum(-(-int(x) // wl.page_size) for x in stored))
    b = {
        "keys": int(stored.sum()) * wl.row_bytes,
        "q": real * wl.heads * wl.head_dim * 2,
        "w": real * wl.heads * 4,
        "block_table": pages * 4,
        "lengths": wl.num_req * 4 * (1 if wl.decode_lens is None else 2),
    }
    b["scorer"] = sum(b.values())
    b["topk_out"] = wl.num_req * wl.next_n * wl.topk * 4
    b["step"] = b["scorer"] + b["topk_out"]
    return b


def scored_keys_decode(wl, pools=None) -> int:
    """Keys the decode step scores: sum of L over rows with L > k (shorter
    rows are causal-filled without scoring); for a pool selection, over rows
    with more complete pools than pools kept."""
    L, _ = decode_rows(wl)
    if pools is not None:
        B, k = pools[0], pools[1]
        return int(L[L // B > k].sum())
    return int(L[L > wl.topk].sum())


def prefill_plan(wl):
    """Planner chunks with their rows' key counts (per chunk: rec, L array)."""
    import numpy as np
    import sparse_attention_indexer_decode_amd as idx
    recs = idx.idx_prefill_chunks(wl.seq_lens // wl.compress_ratio if wl.compress_ratio > 1 else wl.seq_lens,
                                  wl.query_lens, PREFILL_WORKSPACE_TOKENS, PREFILL_LOGITS_BYTES)
    qstart = np.concatenate([[0], np.cumsum(wl.query_lens.astype(np.int64))])
    out = []
    for rec in recs:
        Ls = []
        for b in range(rec["req_begin"], rec["req_end"]):
            qs = int(wl.query_lens[b])
            off = int(qstart[b] - qstart[rec["req_begin"]])
            lo, hi = max(0, rec["q_begin"] - off), min(qs, rec["q_end"] - off)
            j = np.arange(lo, hi, dtype=np.int64)
            Ls.append((int(wl.seq_lens[b]) - qs + j + 1) // wl.compress_ratio)
        out.append((rec, np.concatenate(Ls) if Ls else np.zeros(0, np.int64)))
    return out


# ---------------------------------------------------------------------------
# Host facts and the CPU baseline
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    """Threads the oracle's numpy (BLAS) uses on this host."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline_decode(wl, budget_s: float, pools=None) -> dict:
    """The oracle on whole requests of the batch in order (cycling) for about
    `budget_s` seconds: dequantise, fp64 logits, top-k (or the pool
    selection)."""
    import oracle
    keys = rows = done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = done % wl.num_req
        lg = oracle.pipeline.decode_logits(wl, requests=[b])
        if pools is None:
            oracle.pipeline.decode_topk(wl, lg, requests=[b])
            keys += int(sum(len(v) for v in lg.values() if len(v) > wl.topk))
        else:
            oracle.pipeline.decode_pool_topk(wl, *pools, logits_by_row=lg, requests=[b])
            keys += int(sum(len(v) for v in lg.values() if len(v) // pools[0] > pools[1]))
        rows += int(sum(1 for v in lg.values() if len(v)))
        done += 1
    dt = time.perf_counter() - t0
    return {"value": keys / dt, "unit": "keys/s", "rows_per_s": rows / dt, "cores": oracle_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{done} requests of the {wl.num_req}-request batch in order, cycling "
                      f"({done / wl.num_req:.2f} passes, {keys} keys scored, {rows} rows, {dt:.1f} s)"}


def prefill_sample_rows(M: int):
    """The first, the last and every 64th row of a chunk."""
    return sorted(set(range(0, M, 64)) | {M - 1}) if M else []


def cpu_baseline_prefill(wl, plan, budget_s: float) -> dict:
    """The oracle on the sampled rows of the chunks, chunk by chunk in plan
    order, until about `budget_s` seconds: the chunk's keys dequantised once,
    each sampled row's fp64 logits, then its top-k."""
    import oracle
    keys = rows = 0
    t0 = time.perf_counter()
    chunks_done = 0
    for rec, L in plan:
        sample = prefill_sample_rows(len(L))
        lg = oracle.pipeline.prefill_chunk_logits(wl, rec, sample_rows=sample)
        for r in sample:
            oracle.topk.topk_row(lg[r], int(L[r]), wl.topk)
            keys += int(L[r]) if L[r] > wl.topk else 0
            rows += 1
        chunks_done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": keys / dt, "unit": "keys/s", "rows_per_s": rows / dt, "cores": oracle_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{rows} rows: the first, the last and every 64th row of each of the first {chunks_done} "
                      f"of {len(plan)} chunks, {keys} keys scored, {dt:.1f} s"}


# ---------------------------------------------------------------------------
# Committed counter profiles -> traffic
# ---------------------------------------------------------------------------

def profile_name(cfg: str) -> str:
    return {"C1": "score_kernel_fp8_decode_tiny_c1", "C2": "score_kernel_fp8_decode_32req",
            "C3": "score_kernel_fp8_decode_mtp_c3", "C4": "score_kernel_mxfp4_decode_c4",
            "C5": "score_block_kernel_fp8_prefill", "V4": "score_kernel_fp8_decode_compressed_v4",
            "P2": "score_kernel_fp8_decode_pool_p2"}[cfg]


def load_traffic(cfg: str):
    """HBM bytes per launch of the dominant kernel from its committed counter
    summary, or None unless it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", profile_name(cfg) + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    if prof.get("source_hash") != kernel_source_hash() or prof.get("workload") != cfg:
        return None
    return prof.get("traffic_bytes_per_launch")


# ---------------------------------------------------------------------------
# Timing helpers
# ---------------------------------------------------------------------------

def event_ms(stream, fn, n: int) -> float:
    """Mean duration per call of n back-to-back calls of fn(i) between two
    HIP events on `stream`."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def wall_ms(fn, n: int) -> float:
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / n


def capture(fn, n_inner: int):
    """A HIP graph of fn(0) .. fn(n_inner - 1) captured on a side stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        for i in range(n_inner):
            fn(i)
    torch.cuda.synchronize()
    return g


# ---------------------------------------------------------------------------
# Decode and prefill runs
# ---------------------------------------------------------------------------

def calib_copy(args, dev) -> None:
    """A plain elementwise copy of known size, for scaling the HBM counters."""
    import torch

    src = torch.ones((args.calib_mib << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def run_decode(wl, args, pools=None) -> dict:
    import numpy as np
    import torch

    import sparse_attention_indexer_decode_amd as idx

    dev = torch.device("cuda:0")
    copies = args.copies if args.copies else DEFAULT_COPIES.get(wl.name, 2)
    pool_copies = [torch.from_numpy(wl.cache).to(dev)]
    for _ in range(copies - 1):
        pool_copies.append(pool_copies[0].clone())
    caches = [idx.Cache(p, wl.head_dim, wl.fmt, wl.page_size) for p in pool_copies]
    bt = torch.from_numpy(wl.block_table).to(dev)
    seq = torch.from_numpy(wl.seq_lens).to(dev)
    dl = None if wl.decode_lens is None else torch.from_numpy(wl.decode_lens).to(dev)
    rows = idx.Rows.decode(bt, seq, int(wl.seq_lens.max()), next_n=wl.next_n, decode_lens=dl,
                           compress_ratio=wl.compress_ratio)
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wl.w).to(dev)
    k, R = wl.topk, rows.num_rows
    if pools is not None:
        pl = idx.pools(*pools)
        outs = torch.empty((R, (pools[1] + 1) * pools[0]), dtype=torch.int32, device=dev)
        ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_DECODE_POOL_TOPK, caches[0], rows, wl.heads, 0),
                               dev)
    else:
        outs = torch.empty((R, k), dtype=torch.int32, device=dev)
        ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_DECODE_TOPK, caches[0], rows, wl.heads, k), dev)
    ML = int(wl.seq_lens.max()) // wl.compress_ratio
    logits = torch.empty((R, max(-(-ML // 64) * 64, 64)), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        if pools is not None:
            idx.idx_decode_pool_topk(caches[i % copies], rows, q, w, pl, outs, None, ws)
        else:
            idx.idx_decode_topk(caches[i % copies], rows, q, w, k, outs, ws)

    def select(out):
        if pools is not None:
            idx.idx_pool_topk(logits, rows, pl, out, None, ws)
        else:
            idx.idx_topk(logits, rows, k, out, ws)

    if args.calib:
        calib_copy(args, dev)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    first = outs.clone()
    # the two launches called one by one give the same rows
    sep = torch.full_like(outs, -7)
    idx.idx_logits_paged(caches[0], rows, q, w, logits, ws)
    select(sep)
    torch.cuda.synchronize()
    assert torch.equal(first, sep), f"{wl.name}: the one-call decode differs from the scorer + selection calls"

    # timed region: K whole steps back to back, wall clock between syncs
    step_ms = wall_ms(lambda i: step(args.warmup + i), args.steps)
    assert torch.equal(first, outs), f"{wl.name}: decode top-k is not deterministic across steps"

    # the same steps replayed from a HIP graph: one graph holds at least
    # eight steps (cycling the pool copies), so that a replay's own launch
    # cost is spread as it would be in a serving loop
    n_graph = max(copies, 8)
    g = capture(step, n_graph)
    reps = max(1, args.steps // n_graph)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(first, outs), f"{wl.name}: graph replay differs from eager"
    graph_ms = wall_ms(lambda i: g.replay(), reps) / n_graph
    assert torch.equal(first, outs), f"{wl.name}: graph replay differs from eager"

    # per-kernel launch durations: HIP events around back-to-back launches
    # on the launch stream (the scorer on the rotated pools)
    score_ms = event_ms(stream, lambda i: idx.idx_logits_paged(caches[i % copies], rows, q, w, logits, ws),
                        args.steps)
    topk_ms = event_ms(stream, lambda i: select(sep), args.steps)
    torch.cuda.synchronize()
    assert idx.idx_read_device_status(ws) == 0

    keys = scored_keys_decode(wl, pools)
    _, real = decode_rows(wl)
    ab = decode_bytes(wl)
    if pools is not None:   # the output is the expanded positions
        ab["topk_out"] = R * (pools[1] + 1) * pools[0] * 4
        ab["step"] = ab["scorer"] + ab["topk_out"]
    achieved = ab["scorer"] / (score_ms * 1e-3) / 1e9
    step_gbs = ab["step"] / (step_ms * 1e-3) / 1e9
    graph_gbs = ab["step"] / (graph_ms * 1e-3) / 1e9
    res = {
        "value": keys / (step_ms * 1e-3), "unit": "keys/s", "rows_per_s": real / (step_ms * 1e-3),
        "ms_per_step": step_ms, "ms_per_step_graph": graph_ms, "value_graph": keys / (graph_ms * 1e-3),
        "keys_scored": keys, "rows": real, "grid_rows": R, "scorer_ms_avg": score_ms, "topk_ms_avg": topk_ms,
        "pool_copies_rotated": copies,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(wl.name),
                     "algorithmic_bytes_per_launch": ab["scorer"], "launch_ms_avg": score_ms,
                     "kernel": f"{scorer_kernel_name(wl)} (idx_logits_paged: score_kernel<D, MXFP4, M-tiles>)"},
        "whole_step": {"algorithmic_bytes": ab["step"], "achieved": step_gbs, "frac": step_gbs / HBM_PEAK_GBS,
                       "achieved_graph": graph_gbs, "frac_graph": graph_gbs / HBM_PEAK_GBS, "unit": "GB/s"},
    }
    del pool_copies, caches, logits, outs, sep, ws, g
    torch.cuda.empty_cache()
    return res


def run_prefill(wl, args) -> dict:
    import numpy as np
    import torch

    import sparse_attention_indexer_decode_amd as idx

    dev = torch.device("cuda:0")
    cache = idx.Cache(torch.from_numpy(wl.cache).to(dev), wl.head_dim, wl.fmt, wl.page_size)
    bt = torch.from_numpy(wl.block_table).to(dev)
    seq = torch.from_numpy(wl.seq_lens).to(dev)
    qsl = torch.from_numpy(np.concatenate([[0], np.cumsum(wl.query_lens)]).astype(np.int32)).to(dev)
    q = torch.from_numpy(wl.q.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(wl.w).to(dev)
    k = wl.topk
    plan = prefill_plan(wl)
    chunks = []
    for rec, L in plan:
        b0, b1 = rec["req_begin"], rec["req_end"]
        r = idx.Rows.prefill(bt[b0:b1], seq[b0:b1], qsl[b0:b1 + 1], rec["q_begin"], rec["q_end"],
                             int(wl.seq_lens[b0:b1].max()), compress_ratio=wl.compress_ratio)
        M, N = rec["q_end"] - rec["q_begin"], rec["total_seq_lens"]
        chunks.append((r, q[rec["token_begin"]:rec["token_end"]], w[rec["token_begin"]:rec["token_end"]], M, N))
    pairs = int(sum(int(L.sum()) for _, L in plan))
    keys = int(sum(int(L[L > k].sum()) for _, L in plan))
    n_rows = int(sum(len(L) for _, L in plan))
    flops = pairs * 2 * wl.heads * wl.head_dim
    big = max(M * N for _, _, _, M, N in chunks)
    logits_buf = torch.empty(big, dtype=torch.float32, device=dev)
    outs = torch.empty((max(c[3] for c in chunks), k), dtype=torch.int32, device=dev)
    ws_bytes = max(max(idx.idx_workspace_bytes(idx.IDX_OP_LOGITS, cache, c[0], wl.heads, 0),
                       idx.idx_workspace_bytes(idx.IDX_OP_TOPK, None, c[0], 0, k)) for c in chunks)
    ws = idx.new_workspace(ws_bytes, dev)
    stream = torch.cuda.current_stream()
    if args.calib:
        calib_copy(args, dev)

    def score(ci):
        r, qq, ww, M, N = chunks[ci]
        idx.idx_logits_paged(cache, r, qq, ww, logits_buf[: M * N].view(M, N), ws)

    def select(ci):
        r, qq, ww, M, N = chunks[ci]
        idx.idx_topk(logits_buf[: M * N].view(M, N), r, k, outs[:M], ws)

    def one_pass(_i=0):
        for ci in range(len(chunks)):
            score(ci)
            select(ci)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    last = outs.clone()
    step_ms = wall_ms(one_pass, args.steps)
    assert torch.equal(last, outs), "prefill top-k is not deterministic across passes"
    g = capture(one_pass, 1)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(last, outs), "prefill graph replay differs from eager"
    graph_ms = wall_ms(lambda i: g.replay(), max(1, args.steps // 2))
    assert torch.equal(last, outs), "prefill graph replay differs from eager"
    # scorer launches: every chunk's scorer back to back, HIP events, mean per
    # launch (a launch is one chunk); the same for the selector
    nc = len(chunks)
    reps = max(1, args.steps // 4)
    score_ms = event_ms(stream, lambda i: score(i % nc), reps * nc)
    topk_ms = event_ms(stream, lambda i: select(i % nc), reps * nc)
    assert idx.idx_read_device_status(ws) == 0
    per_launch_flops = flops / nc
    tflops = per_launch_flops / (score_ms * 1e-3) / 1e12
    step_tflops = flops / (step_ms * 1e-3) / 1e12
    graph_tflops = flops / (graph_ms * 1e-3) / 1e12
    res = {
        "value": keys / (step_ms * 1e-3), "unit": "keys/s", "rows_per_s": n_rows / (step_ms * 1e-3),
        "ms_per_step": step_ms, "ms_per_step_graph": graph_ms, "value_graph": keys / (graph_ms * 1e-3),
        "keys_scored": keys, "pairs": pairs, "rows": n_rows, "chunks": nc,
        "scorer_ms_avg": score_ms, "scorer_ms_per_pass": score_ms * nc,
        "topk_ms_avg": topk_ms, "topk_ms_per_pass": topk_ms * nc,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / FP8_PEAK_TFLOPS, "traffic": load_traffic(wl.name),
                     "peak_dtype": "fp8 (the method's bar)", "mfma_dtype": "bf16",
                     "peak_bf16": BF16_PEAK_TFLOPS, "frac_bf16": tflops / BF16_PEAK_TFLOPS,
                     "algorithmic_flops_per_launch": per_launch_flops, "launch_ms_avg": score_ms,
                     "kernel": f"{scorer_kernel_name(wl)} (idx_logits_paged on a prefill chunk)"},
        "whole_step": {"algorithmic_flops": flops, "achieved": step_tflops, "frac": step_tflops / FP8_PEAK_TFLOPS,
                       "frac_bf16": step_tflops / BF16_PEAK_TFLOPS, "achieved_graph": graph_tflops,
                       "frac_graph": graph_tflops / FP8_PEAK_TFLOPS, "unit": "TFLOP/s"},
    }
    del logits_buf, outs, ws, g, cache
    torch.cuda.empty_cache()
    return res, plan


def run_all(args):
    import torch

    from workloads import config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    names = [c.strip() for c in args.configs.split(",") if c.strip()]
    per = {}
    for name in names:
        print(f"[bench] {name}: generating", file=sys.stderr, flush=True)
        pools = None
        if name in POOL_WORKLOADS:
            base, *pools = POOL_WORKLOADS[name]
            wl = config(base)
            wl.name = name
        else:
            wl = config(name)
        print(f"[bench] {name}: timing", file=sys.stderr, flush=True)
        if wl.kind == "prefill":
            res, plan = run_prefill(wl, args)
        else:
            res, plan = run_decode(wl, args, pools), None
        if not args.no_cpu_baseline:
            print(f"[bench] {name}: cpu baseline", file=sys.stderr, flush=True)
            budget = CPU_BUDGET_S.get(name, 5.0) * args.cpu_scale
            res["cpu_baseline"] = (cpu_baseline_prefill(wl, plan, budget) if plan is not None
                                   else cpu_baseline_decode(wl, budget, pools))
        res["workload"] = WORKLOADS[name]
        per[name] = res
        print(f"[bench] {name}: {res['value']:.4g} keys/s, step {res['ms_per_step']:.4f} ms, "
              f"{res['roofline']['kernel'].split(' ')[0]} frac {res['roofline']['frac']:.3f}",
              file=sys.stderr, flush=True)
        del wl
    # headline: the largest workload measured (C5 by work, then C4, ...)
    order = ["C5", "C4", "C3", "V4", "C2", "P2", "C1"]
    head = next(n for n in order if n in per)
    h = per[head]
    line = {
        "metric": METRIC, "value": h["value"], "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOADS[head], "name": head},
        "rows_per_s": h["rows_per_s"],
        "roofline": h["roofline"],
        "whole_step": h["whole_step"],
    }
    if "cpu_baseline" in h:
        line["cpu_baseline"] = h["cpu_baseline"]
    line["configs"] = per
    line["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(line), flush=True)


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
        ms = event_ms(stream, lambda i: idx.idx_cache_write(cache, k, slots, ws, stream), args.steps)
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
            while time.perf_counter() - t0 < 2.5 * args.cpu_scale:
                oracle.cache_write.quantize_rows(kb, fmt)
                n += sample
            dt = time.perf_counter() - t0
            res["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s", "cores": oracle_threads(), "kind": "oracle",
                                   "cpu": cpu_model(),
                                   "sample": f"the first {sample} tokens quantised repeatedly ({n} tokens, {dt:.1f} s)"}
        print(json.dumps(res), flush=True)
        del pool


# ---------------------------------------------------------------------------
# rocprofv3 output -> profiles/
# ---------------------------------------------------------------------------

def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize(name, cfg, stats_dir, fetch_dir, write_dir, commands, bench_json=None):
    """Kernel trace and FETCH_SIZE / WRITE_SIZE counters of one workload's
    dominant kernel -> profiles/NAME.{md,json}."""
    import numpy as np

    from workloads import config

    wl = config(POOL_WORKLOADS[cfg][0]) if cfg in POOL_WORKLOADS else config(cfg)
    kname = scorer_kernel_name(wl)
    out = {"workload": cfg, "kernel": kname, "source_hash": kernel_source_hash(), "commands": commands}
    stats = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    lines = []
    for r in _csv_rows(stats[0]):
        if kname in r["Name"]:
            out["calls"] = int(r["Calls"])
            out["avg_ns"] = float(r["AverageNs"])
            out["min_ns"] = float(r["MinNs"])
            out["max_ns"] = float(r["MaxNs"])
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")

    def counter(d, cname):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        per_kernel, copy_vals = [], []
        for r in _csv_rows(files[0]):
            if r.get("Counter_Name") != cname:
                continue
            v = float(r["Counter_Value"])
            kn = r.get("Kernel_Name", "")
            if kname in kn:
                per_kernel.append(v)
            elif CALIB_SUBSTR in kn:
                copy_vals.append(v)
        return per_kernel, copy_vals

    fetch, fcopy = counter(fetch_dir, "FETCH_SIZE")
    write, wcopy = counter(write_dir, "WRITE_SIZE")
    calib_bytes = 256 << 20
    f_scale = calib_bytes / (np.median(fcopy) * 1024) if fcopy else 1.0
    w_scale = calib_bytes / (np.median(wcopy) * 1024) if wcopy else 1.0
    out.update(fetch_kib_per_launch=float(np.median(fetch)) if fetch else None,
               write_kib_per_launch=float(np.median(write)) if write else None,
               copy_fetch_kib=float(np.median(fcopy)) if fcopy else None,
               copy_write_kib=float(np.median(wcopy)) if wcopy else None,
               fetch_scale=f_scale, write_scale=w_scale)
    if fetch and write:
        out["traffic_bytes_per_launch"] = (out["fetch_kib_per_launch"] * f_scale
                                           + out["write_kib_per_launch"] * w_scale) * 1024
    if wl.kind == "prefill":
        out["algorithmic"] = "flops per launch: 2 H D per (row, key) pair of the chunk (the bench line)"
    else:
        out["algorithmic_bytes_per_launch"] = decode_bytes(wl)["scorer"]
    bl = None
    if bench_json:
        with open(bench_json) as f:
            bl = json.loads(f.read().strip().splitlines()[-1])
        c = bl["configs"][cfg]
        out["bench_scorer_ms_avg"] = c["scorer_ms_avg"]
        out["bench_topk_ms_avg"] = c["topk_ms_avg"]
        out["bench_roofline"] = c["roofline"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", name + ".json"), "w") as f:
        json.dump(out, f, indent=1)
    md = [f"# {kname} on {cfg}: {WORKLOADS[cfg]}", "",
          "Commands (run from the repository root on one MI355X):", ""]
    md += [f"    {c}" for c in commands]
    md += ["", "## rocprofv3 --kernel-trace --stats", "",
           "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"] + lines
    if bl is not None:
        c = bl["configs"][cfg]
        rf = c["roofline"]
        md += ["", "## HIP-event launch durations in the benchmark (mean per launch, back-to-back launches)", "",
               f"- scorer {c['scorer_ms_avg'] * 1e3:.2f} us per launch (rocprofv3 average "
               f"{out.get('avg_ns', float('nan')) / 1e3:.2f} us)",
               f"- selector {c['topk_ms_avg'] * 1e3:.2f} us per launch",
               f"- step {c['ms_per_step'] * 1e3:.2f} us eager, {c['ms_per_step_graph'] * 1e3:.2f} us from a HIP graph; "
               f"{c['value']:.4g} keys/s",
               f"- roofline: {rf['achieved']:.1f} {rf['unit']} = {rf['frac'] * 100:.1f} % of {rf['peak']:.0f} {rf['unit']}"]
    md += ["", "## HBM traffic of the kernel (rocprofv3 --pmc, per dispatch, median)", "",
           f"- FETCH_SIZE {out['fetch_kib_per_launch']} KiB, WRITE_SIZE {out['write_kib_per_launch']} KiB",
           f"- a plain 256 MiB fp32 copy reads as FETCH {out['copy_fetch_kib']} KiB / WRITE {out['copy_write_kib']} KiB "
           f"-> scale {f_scale:.4f} / {w_scale:.4f}",
           f"- traffic per launch {out.get('traffic_bytes_per_launch')} B"
           + (f" vs algorithmic {out['algorithmic_bytes_per_launch']} B" if "algorithmic_bytes_per_launch" in out
              else ""),
           f"- kernel source hash {out['source_hash']}"]
    with open(os.path.join(ROOT, "profiles", name + ".md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--configs", default=",".join(ALL_CONFIGS), help="comma-separated workloads (C1..C5, V4)")
    ap.add_argument("--config", default=None, help="a single workload (same as --configs X)")
    ap.add_argument("--copies", type=int, default=0, help="rotated decode pool copies (0 = per-workload default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-scale", type=float, default=1.0, help="scales every CPU-baseline time budget")
    ap.add_argument("--calib", action="store_true", help="also run a plain copy for counter scaling")
    ap.add_argument("--calib-mib", type=int, default=256)
    ap.add_argument("--summarize", nargs=5, metavar=("NAME", "CONFIG", "STATS_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--commands", nargs="*", default=[])
    ap.add_argument("--bench-json", default=None)
    ap.add_argument("--cache-write", action="store_true", help="measure the index-cache write instead")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize, args.commands, args.bench_json)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; --gpus must be 1 (the multi-GPU sharding is "
                                   "described, not implemented)"}), flush=True)
        sys.exit(2)
    if args.config:
        args.configs = args.config
    if args.cache_write:
        run_cache_write(args)
        return
    run_all(args)


if __name__ == "__main__":
    main()
