"""GPU: idx_decode_topk_noalloc (no workspace, the library's static scratch)
against idx_decode_topk (caller workspace), through the C ABI.

Two calls in a row on the same GPU, the second with a smaller batch, each
bit-exact against the workspace entry point (the same kernels run on the same
logits, so the rows are identical); a block-table entry outside the pool
reaches the caller's status word; a batch that needs more than the static
scratch is refused before anything is enqueued.
"""

import numpy as np
import pytest
import torch

import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import Dev
from workloads import build_decode

pytestmark = pytest.mark.gpu


def _pair(wl, status=None):
    dev = Dev(wl)
    ref, _ = dev.decode_topk()
    rows = dev.decode_rows()
    out = torch.full((rows.num_rows, wl.topk), -7, dtype=torch.int32, device=dev.device)
    print(f"noalloc: {wl.name} rows {rows.num_rows} max L {int(wl.seq_lens.max())} k {wl.topk}", flush=True)
    idx.idx_decode_topk_noalloc(dev.cache, rows, dev.q, dev.w, wl.topk, out, status)
    torch.cuda.synchronize()
    return ref, out.cpu().numpy()


def test_noalloc_matches_workspace_two_calls():
    rng = np.random.default_rng(808)
    # first call: 24 requests, next_n 2 with short requests, rows past 32768
    # keys (the split selector with chunk candidates in the scratch)
    seq1 = rng.integers(100, 70000, size=24).astype(np.int32)
    seq1[:3] = [2047, 2049, 69999]
    dl1 = rng.integers(1, 3, size=24).astype(np.int32)
    wl1 = build_decode(seed=809, seq_lens=seq1, heads=64, head_dim=128, topk=2048, next_n=2, decode_lens=dl1,
                       name="noalloc-1")
    ref1, got1 = _pair(wl1)
    assert np.array_equal(ref1, got1)
    # second call: a smaller batch (fewer, shorter rows) reusing the scratch
    seq2 = rng.integers(1, 9000, size=5).astype(np.int32)
    wl2 = build_decode(seed=810, seq_lens=seq2, heads=32, head_dim=64, topk=256, name="noalloc-2")
    ref2, got2 = _pair(wl2)
    assert np.array_equal(ref2, got2)
    # the first batch again after the smaller one: the same rows
    _, again = _pair(wl1)
    assert np.array_equal(ref1, again)


def test_noalloc_status_word_and_mxfp4():
    seq = np.array([5000, 130, 64, 1], dtype=np.int32)
    wl = build_decode(seed=811, seq_lens=seq, heads=64, head_dim=128, topk=64, fmt="mxfp4", name="noalloc-mx")
    dev = torch.device("cuda")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ref, got = _pair(wl, status)
    assert np.array_equal(ref, got)
    assert int(status.item()) == 0
    # a block-table entry outside the pool: flagged in the caller's word
    wl.block_table = wl.block_table.copy()
    wl.block_table[0, 3] = wl.num_pages + 5
    d = Dev(wl)
    rows = d.decode_rows()
    out = torch.full((rows.num_rows, wl.topk), -7, dtype=torch.int32, device=dev)
    idx.idx_decode_topk_noalloc(d.cache, rows, d.q, d.w, wl.topk, out, status)
    torch.cuda.synchronize()
    assert int(status.item()) == idx.IDX_DEV_BAD_PAGE
    # rows 1..3 do not touch the bad entry: same as the workspace path
    ref2, _ = d.decode_topk()
    assert np.array_equal(out.cpu().numpy()[1:], ref2[1:])


def test_noalloc_refuses_rows_beyond_scratch():
    dev = torch.device("cuda")
    R = 400                        # 400 rows x 131072 keys of fp32 logits > 160 MiB
    bt = torch.zeros((R, 2048), dtype=torch.int32, device=dev)
    seq = torch.full((R,), 131072, dtype=torch.int32, device=dev)
    rows = idx.Rows.decode(bt, seq, 131072)
    pool = torch.zeros((4, 64 * 132), dtype=torch.uint8, device=dev)
    cache = idx.Cache(pool, 128, "fp8")
    q = torch.zeros((R, 64, 128), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((R, 64), dtype=torch.float32, device=dev)
    out = torch.full((R, 2048), -7, dtype=torch.int32, device=dev)
    with pytest.raises(idx.IdxError) as e:
        idx.idx_decode_topk_noalloc(cache, rows, q, w, 2048, out)
    assert e.value.status == 3                     # IDX_ENOSPC
    torch.cuda.synchronize()
    assert (out == -7).all()                      # nothing ran
