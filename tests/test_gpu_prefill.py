"""GPU parity of the prefill path: the planner's chunks scored by
idx_logits_paged on PREFILL rows (columns at each request's workspace
offset ks), then idx_topk on the chunk's logits."""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import Dev, check_logits, check_topk_e2e, fp32_rows, topk_workspace
from workloads import build_prefill

pytestmark = pytest.mark.gpu


def _chunks(wl, ws_tokens, budget):
    recs = idx.idx_prefill_chunks(wl.seq_lens, wl.query_lens, ws_tokens, budget)
    ref = oracle.planner.chunk_records(wl.seq_lens, wl.query_lens, ws_tokens, budget)
    assert [{f: r[f] for f in ref[0]} for r in recs] == ref if ref else not recs
    return recs


def _run_chunk(dev, rec):
    """GPU logits [M, N] (NaN where not written) and top-k rows of a chunk."""
    wl = dev.wl
    rows = dev.prefill_rows(rec)
    M, N = rec["q_end"] - rec["q_begin"], rec["total_seq_lens"]
    q, w = dev.chunk_queries(rec)
    logits = torch.full((M, N), float("nan"), device=dev.device)
    ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_LOGITS, dev.cache, rows, wl.heads, 0), dev.device)
    idx.idx_logits_paged(dev.cache, rows, q, w, logits, ws)
    out = torch.full((M, wl.topk), -7, dtype=torch.int32, device=dev.device)
    idx.idx_topk(logits, rows, wl.topk, out, topk_workspace(rows, wl.topk, dev.device))
    torch.cuda.synchronize()
    assert idx.idx_read_device_status(ws) == 0
    return logits.cpu().numpy(), out.cpu().numpy(), rows


CASES = [
    # seq_lens, query_lens, workspace tokens, logits budget (bytes), fmt, heads, head_dim, k
    ([300, 1000, 0, 777, 64], [100, 200, 0, 50, 64], 1200, 200 * 1024, "fp8", 64, 128, 128),
    ([2000, 65, 129], [700, 65, 1], 2100, 1 << 20, "fp8", 32, 64, 64),
    ([1500, 900], [1500, 300], 4096, 1 << 22, "mxfp4", 64, 128, 256),
    ([4000], [600], 4000, 4000 * 4 * 150, "fp8", 17, 32, 100),   # one request, sub-chunked on M
    # one long request among short ones: most workgroups get one or two pages,
    # and ranges start and end inside groups of every size
    ([5000, 70, 65, 1, 130, 64], [8, 8, 3, 1, 20, 64], 6000, 1 << 22, "fp8", 64, 128, 32),
    # a chunk of fewer than 512 rows with rows past 32768 keys: the selector
    # splits those rows over workgroups and merges them
    ([40000, 300], [64, 16], 41000, 1 << 26, "fp8", 16, 64, 256),
    # the same with the long rows' logits at an odd column offset (their
    # keys start after the short request's 301), so the split reads rows
    # that are not 16-byte aligned
    ([301, 40000], [16, 64], 41000, 1 << 26, "fp8", 16, 64, 256),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_chunks_logits_and_topk(case):
    seq, ql, ws_tokens, budget, fmt, H, D, k = CASES[case]
    wl = build_prefill(seed=200 + case, seq_lens=seq, query_lens=ql, heads=H, head_dim=D, topk=k, fmt=fmt,
                       name=f"prefill-{case}")
    recs = _chunks(wl, ws_tokens, budget)
    print(f"case {case}: {len(recs)} chunks {recs}", flush=True)
    assert len(recs) >= 2 or case >= 3
    dev = Dev(wl)
    for ci, rec in enumerate(recs):
        got, out, rows = _run_chunk(dev, rec)
        req, j, L, ks, _ = oracle.pipeline.prefill_chunk_row_info(wl, rec)
        ref = oracle.pipeline.prefill_chunk_logits(wl, rec)
        check_logits(got, ref, col0=ks, label=f"case {case} chunk {ci}")
        # the top-k indices are key positions within each row's request
        check_topk_e2e(out, ref, L, k, label=f"case {case} chunk {ci}")
        # and bit-exact on the oracle's fp32 logits
        buf = fp32_rows(ref, got.shape[0], got.shape[1], col0=ks)
        o2 = torch.full((got.shape[0], k), -7, dtype=torch.int32, device=dev.device)
        idx.idx_topk(torch.from_numpy(buf).to(dev.device), rows, k, o2, topk_workspace(rows, k, dev.device))
        o2 = o2.cpu().numpy()
        for r in range(got.shape[0]):
            exp = oracle.topk.topk_row(buf[r, ks[r] : ks[r] + L[r]].astype(np.float64), int(L[r]), k)
            assert np.array_equal(o2[r], exp), f"case {case} chunk {ci} row {r}"
