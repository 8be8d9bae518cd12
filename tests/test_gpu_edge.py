"""GPU behaviour of degenerate decode batches, through the C ABI: requests
with no keys, batches whose rows are all padding, lengths beyond the host
bound (clamped into [0, max_seq_len], as the header states) and a batch of no
requests.  Expected values come from the oracle on the clamped lengths, or
are the method's fixed outputs for rows without keys (all -1, no logit
written)."""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import Dev, check_logits, check_topk_e2e, topk_workspace
from workloads import build_decode

pytestmark = pytest.mark.gpu


def _untouched_and_empty(dev, n_rows, k):
    logits, _ = dev.logits_decode()
    assert np.isnan(logits).all(), "a logit was written for a row without keys"
    out, _ = dev.decode_topk()
    assert out.shape == (n_rows, k) and (out == -1).all()
    rows = dev.decode_rows()
    got = torch.full((n_rows, k), -7, dtype=torch.int32, device=dev.device)
    lg = torch.from_numpy(logits).to(dev.device)
    idx.idx_topk(lg, rows, k, got, topk_workspace(rows, k))
    torch.cuda.synchronize()
    assert (got.cpu().numpy() == -1).all()


def test_every_request_empty():
    wl = build_decode(seed=72, seq_lens=[0, 0, 0], heads=64, head_dim=128, topk=64, fmt="fp8", name="empty")
    print(f"case {wl.name}", flush=True)
    _untouched_and_empty(Dev(wl), 3, 64)


def test_every_row_padded():
    wl = build_decode(seed=73, seq_lens=[500, 70], heads=32, head_dim=128, topk=64, fmt="fp8", next_n=2,
                      decode_lens=np.zeros(2, np.int32), name="padded")
    print(f"case {wl.name}", flush=True)
    _untouched_and_empty(Dev(wl), 4, 64)


def test_lengths_clamped_to_the_host_bound():
    """seq_lens 5000 and -7 with max_seq_len 1000 score like 1000 and 0: the
    oracle on the clamped lengths, nothing written past column 1000 (the
    next row's first columns stay NaN) and the block table read only as far
    as the bound."""
    wl = build_decode(seed=71, seq_lens=[1000, 300, 0], heads=64, head_dim=128, topk=256, fmt="fp8",
                      name="clamped")
    print(f"case {wl.name}", flush=True)
    dev = Dev(wl)
    assert dev.max_len == 1000
    dev.seq = torch.tensor([5000, 300, -7], dtype=torch.int32, device=dev.device)
    ref = oracle.pipeline.decode_logits(wl)
    L, _ = oracle.pipeline.decode_row_info(wl)
    got, _ = dev.logits_decode()
    assert got.shape[1] == 1000
    check_logits(got, {r: v for r, v in ref.items() if len(v)}, label=wl.name)
    assert np.isnan(got[2]).all()
    out, _ = dev.decode_topk()
    check_topk_e2e(out, ref, L, wl.topk, label=wl.name)


def test_no_requests():
    d = torch.device("cuda")
    pool = torch.zeros((1, 64 * 132), dtype=torch.uint8, device=d)
    cache = idx.Cache(pool, 128, "fp8")
    bt = torch.zeros((0, 1), dtype=torch.int32, device=d)
    seq = torch.zeros((0,), dtype=torch.int32, device=d)
    rows = idx.Rows.decode(bt, seq, 64)
    assert rows.num_rows == 0
    q = torch.zeros((1, 64, 128), dtype=torch.bfloat16, device=d)
    w = torch.zeros((1, 64), dtype=torch.float32, device=d)
    out = torch.full((1, 16), -7, dtype=torch.int32, device=d)
    ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_DECODE_TOPK, cache, rows, 64, 16), d)
    idx.idx_decode_topk(cache, rows, q, w, 16, out, ws)
    logits = torch.full((1, 64), float("nan"), device=d)
    idx.idx_logits_paged(cache, rows, q, w, logits, ws)
    torch.cuda.synchronize()
    assert (out.cpu() == -7).all() and torch.isnan(logits.cpu()).all()
