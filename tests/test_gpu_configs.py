"""GPU parity on the five named workloads at full size, in the launch
configuration the benchmark times.

C1, C2: every row (logits, top-k on the GPU's logits end to end, top-k on
        the oracle's fp32 logits bit-exact, idx_decode_topk end to end).
C3, C4: the GPU runs the whole batch; the oracle checks a sample of
        requests one by one (short, long, padded, causal-fill), and the
        invariants are checked on every row.  The same for V4, the
        compressed-cache decode (64 x 131072 tokens at ratio 4, 256-token
        pages).
C5:     the planner's 16 chunks; per chunk the GPU scores and selects all
        rows, the oracle checks sampled rows, invariants on every row.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import Dev, check_logits, check_topk_e2e, fp32_rows, topk_workspace
from workloads import config

pytestmark = pytest.mark.gpu


def check_topk_invariants(out: np.ndarray, L: np.ndarray, k: int, label=""):
    """Every row: ascending unique indices < L, min(L, k) of them, -1 tail,
    the causal fill when L <= k."""
    n = np.minimum(L, k)
    valid = out >= 0
    cnt = valid.sum(axis=1)
    assert np.array_equal(cnt, n), f"{label}: wrong index counts in rows {np.nonzero(cnt != n)[0][:8]}"
    pos = np.arange(k)[None, :]
    assert (valid == (pos < n[:, None])).all(), f"{label}: -1 padding not at the tail"
    for r in range(out.shape[0]):
        v = out[r, : n[r]]
        assert (np.diff(v) > 0).all(), f"{label} row {r}: not ascending"
        if n[r]:
            assert v[-1] < L[r], f"{label} row {r}: index >= L"
        if L[r] <= k:
            assert np.array_equal(v, np.arange(L[r])), f"{label} row {r}: not the causal fill"


def _decode_full(name):
    wl = config(name)
    dev = Dev(wl)
    got, _ = dev.logits_decode()
    out, ws = dev.decode_topk()
    assert idx.idx_read_device_status(ws) == 0
    L, _ = oracle.pipeline.decode_row_info(wl)
    check_topk_invariants(out, L, wl.topk, label=name)
    return wl, dev, got, out, L


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_decode_config_every_row(name):
    wl, dev, got, out, L = _decode_full(name)
    ref = oracle.pipeline.decode_logits(wl)
    check_logits(got, ref, label=name)
    check_topk_e2e(out, ref, L, wl.topk, label=name)
    # top-k on the oracle's fp32 logits: bit-exact
    R = len(L)
    buf = fp32_rows(ref, R, got.shape[1])
    o2 = torch.full((R, wl.topk), -7, dtype=torch.int32, device=dev.device)
    idx.idx_topk(torch.from_numpy(buf).to(dev.device), dev.decode_rows(), wl.topk, o2,
                 topk_workspace(dev.decode_rows(), wl.topk))
    o2 = o2.cpu().numpy()
    for r in range(R):
        exp = oracle.topk.topk_row(buf[r, : L[r]].astype(np.float64), int(L[r]), wl.topk)
        assert np.array_equal(o2[r], exp), f"{name} row {r}"


def _sample_requests(wl, n):
    """Shortest, longest, a request with a padded row (if any) and evenly
    spread others."""
    order = np.argsort(wl.seq_lens, kind="stable")
    pick = {int(order[0]), int(order[-1])}
    if wl.decode_lens is not None:
        short = np.nonzero(wl.decode_lens < wl.next_n)[0]
        if len(short):
            pick.add(int(short[0]))
        pick.update(int(b) for b in np.nonzero(wl.seq_lens <= wl.topk)[0][:1])
    for b in np.linspace(0, wl.num_req - 1, n).astype(int):
        pick.add(int(order[b]))
    return sorted(pick)


@pytest.mark.parametrize("name,n", [("C3", 10), ("C4", 3), ("V4", 3)])
def test_decode_config_sampled(name, n):
    wl, dev, got, out, L = _decode_full(name)
    reqs = _sample_requests(wl, n)
    print(f"{name}: oracle on requests {reqs}", flush=True)
    ref = oracle.pipeline.decode_logits(wl, requests=reqs)
    live = {r: v for r, v in ref.items() if len(v)}
    check_logits(got, live, label=name)
    sel = sorted(ref)
    check_topk_e2e(out[sel], {i: ref[r] for i, r in enumerate(sel)}, L[sel], wl.topk, label=name)
    # padded rows: nothing written, all -1
    for r in np.nonzero(L == 0)[0]:
        assert np.isnan(got[r]).all() and (out[r] == -1).all()


def test_prefill_c5_chunks_sampled():
    wl = config("C5")
    recs = idx.idx_prefill_chunks(wl.seq_lens, wl.query_lens, 65536, 512 << 20)
    assert len(recs) == 16
    dev = Dev(wl)
    rng = np.random.default_rng(55)
    for ci, rec in enumerate(recs):
        rows = dev.prefill_rows(rec)
        M, N = rec["q_end"] - rec["q_begin"], rec["total_seq_lens"]
        q, w = dev.chunk_queries(rec)
        logits = torch.empty((M, N), device=dev.device)
        ws = topk_workspace(rows, wl.topk)
        idx.idx_logits_paged(dev.cache, rows, q, w, logits, ws)
        out = torch.full((M, wl.topk), -7, dtype=torch.int32, device=dev.device)
        idx.idx_topk(logits, rows, wl.topk, out, ws)
        torch.cuda.synchronize()
        assert idx.idx_read_device_status(ws) == 0
        req, j, L, ks, _ = oracle.pipeline.prefill_chunk_row_info(wl, rec)
        outc = out.cpu().numpy()
        check_topk_invariants(outc, L, wl.topk, label=f"C5 chunk {ci}")
        sample = sorted({0, M - 1, *rng.integers(0, M, size=2).tolist()})
        ref = oracle.pipeline.prefill_chunk_logits(wl, rec, sample_rows=sample)
        got = logits[sample].cpu().numpy()
        check_logits(got, {i: ref[r] for i, r in enumerate(sample)}, col0=ks[sample], check_untouched=False,
                     label=f"C5 chunk {ci}")
        check_topk_e2e(outc[sample], {i: ref[r] for i, r in enumerate(sample)}, L[sample], wl.topk,
                       label=f"C5 chunk {ci}")
        print(f"C5 chunk {ci} ok (rows {sample})", flush=True)
        del logits, out
