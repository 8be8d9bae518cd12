"""GPU parity of the compressed index cache (DeepSeek-V4 variant: 256-token
pages, every row's key count divided by the compress ratio) against the CPU
oracle, through the C ABI: decode logits and top-k, prefill chunks."""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import Dev, check_logits, check_topk_e2e, fp32_rows, topk_workspace
from workloads import build_decode, build_prefill

pytestmark = pytest.mark.gpu

# compressed lengths 0, 0, 1, 1, 63, 256, 257, 1250, 5000 at ratio 4
SEQS = [1, 3, 4, 5, 255, 1024, 1029, 5000, 20000]

DECODE_CASES = [
    # fmt, head_dim, heads, next_n, page_size, ratio, k
    ("fp8", 128, 64, 1, 256, 4, 64),
    ("fp8", 128, 64, 2, 256, 4, 512),
    ("fp8", 64, 16, 3, 256, 2, 64),
    ("mxfp4", 128, 64, 2, 256, 4, 64),
    ("fp8", 128, 64, 1, 64, 4, 64),      # ratio on 64-token pages
    ("fp8", 128, 32, 2, 256, 1, 100),    # 256-token pages, no compression
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_compressed_decode(case):
    fmt, D, H, nn, ps, r, k = case
    seed = 700 + DECODE_CASES.index(case)
    rng = np.random.default_rng(seed)
    dl = None
    if nn > 1:
        dl = rng.integers(0, nn + 1, size=len(SEQS)).astype(np.int32)
        dl[-1] = nn
        dl = np.minimum(dl, SEQS).astype(np.int32)
    wl = build_decode(seed=seed, seq_lens=SEQS, heads=H, head_dim=D, topk=k, fmt=fmt, next_n=nn,
                      decode_lens=dl, page_size=ps, compress_ratio=r, name=f"v4-{fmt}-p{ps}-r{r}")
    print(f"case {case} dl={dl}", flush=True)
    dev = Dev(wl)
    ref = oracle.pipeline.decode_logits(wl)
    got, ws = dev.logits_decode()
    check_logits(got, {row: v for row, v in ref.items() if len(v)}, label=wl.name)
    L, _ = oracle.pipeline.decode_row_info(wl)
    for row in np.nonzero(L == 0)[0]:
        assert np.isnan(got[row]).all()
    assert idx.idx_read_device_status(ws) == 0
    out, _ = dev.decode_topk()
    check_topk_e2e(out, ref, L, k, label=wl.name)
    # selection bit-exact on the oracle's fp32 logits
    rows = dev.decode_rows()
    buf = fp32_rows(ref, got.shape[0], got.shape[1])
    o2 = torch.full((got.shape[0], k), -7, dtype=torch.int32, device=dev.device)
    idx.idx_topk(torch.from_numpy(buf).to(dev.device), rows, k, o2, topk_workspace(rows, k, dev.device))
    o2 = o2.cpu().numpy()
    for row in range(got.shape[0]):
        exp = oracle.topk.topk_row(buf[row, : L[row]].astype(np.float64), int(L[row]), k)
        assert np.array_equal(o2[row], exp), f"{wl.name} row {row}"


PREFILL_CASES = [
    # seq_lens, query_lens, workspace tokens (compressed), budget, fmt, heads, head_dim, k, page, ratio
    ([1200, 4000, 0, 777, 256], [100, 200, 0, 50, 64], 900, 64 * 1024, "fp8", 64, 128, 128, 256, 4),
    ([6000, 300], [1500, 300], 4096, 1 << 22, "mxfp4", 64, 128, 256, 256, 4),
    ([4000], [600], 2000, 2000 * 4 * 150, "fp8", 17, 64, 100, 256, 2),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_compressed_prefill(case):
    seq, ql, ws_tokens, budget, fmt, H, D, k, ps, r = PREFILL_CASES[case]
    wl = build_prefill(seed=800 + case, seq_lens=seq, query_lens=ql, heads=H, head_dim=D, topk=k, fmt=fmt,
                       page_size=ps, compress_ratio=r, name=f"v4-prefill-{case}")
    # the planner sees compressed lengths, as the page's builder passes them
    recs = idx.idx_prefill_chunks(wl.seq_lens // r, wl.query_lens, ws_tokens, budget)
    ref_recs = oracle.planner.chunk_records(wl.seq_lens // r, wl.query_lens, ws_tokens, budget)
    assert [{f: x[f] for f in ref_recs[0]} for x in recs] == ref_recs
    print(f"case {case}: {len(recs)} chunks", flush=True)
    dev = Dev(wl)
    for ci, rec in enumerate(recs):
        rows = dev.prefill_rows(rec)
        M, N = rec["q_end"] - rec["q_begin"], rec["total_seq_lens"]
        q, w = dev.chunk_queries(rec)
        logits = torch.full((M, N), float("nan"), device=dev.device)
        ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_LOGITS, dev.cache, rows, wl.heads, 0),
                               dev.device)
        idx.idx_logits_paged(dev.cache, rows, q, w, logits, ws)
        out = torch.full((M, k), -7, dtype=torch.int32, device=dev.device)
        idx.idx_topk(logits, rows, k, out, topk_workspace(rows, k, dev.device))
        torch.cuda.synchronize()
        assert idx.idx_read_device_status(ws) == 0
        got = logits.cpu().numpy()
        req, j, L, ks, _ = oracle.pipeline.prefill_chunk_row_info(wl, rec)
        ref = oracle.pipeline.prefill_chunk_logits(wl, rec)
        check_logits(got, ref, col0=ks, label=f"case {case} chunk {ci}")
        check_topk_e2e(out.cpu().numpy(), ref, L, k, label=f"case {case} chunk {ci}")
