"""GPU parity on the five named workloads at full size, in the launch
configuration the benchmark times.

C1, C2, C3, C4 and V4 (the compressed-cache decode, 64 x 131072 tokens at
ratio 4 on 256-token pages): every row -- logits against the oracle,
idx_decode_topk end to end against the oracle's logits, and idx_topk on the
oracle's fp32-rounded logits bit-exact, with the batch's own row descriptor
(so the same selector kernels as the benchmark run).  The large workloads
are checked in request groups so that each test stays short; the GPU runs
each workload once per module.

C5: the planner's 16 chunks; per chunk the GPU scores and selects every row
and the invariants are checked on every row; the oracle checks the first,
the last and every 64th row of each chunk (528 rows): logits, top-k end to
end, and idx_topk bit-exact on the chunk's logits with those rows replaced
by the oracle's fp32 values.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import Dev, check_logits, check_topk_e2e, topk_workspace
from workloads import config

pytestmark = pytest.mark.gpu

_RUNS = {}


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


def _decode_run(name):
    """The workload on the GPU once: logits (NaN-poisoned buffer), fused
    decode top-k, invariants on every row."""
    if name not in _RUNS:
        print(f"{name}: generating and running on the GPU", flush=True)
        wl = config(name)
        dev = Dev(wl)
        got, _ = dev.logits_decode()
        out, ws = dev.decode_topk()
        assert idx.idx_read_device_status(ws) == 0
        L, _ = oracle.pipeline.decode_row_info(wl)
        check_topk_invariants(out, L, wl.topk, label=name)
        for r in np.nonzero(L == 0)[0]:          # padded rows: nothing written, all -1
            assert np.isnan(got[r]).all() and (out[r] == -1).all()
        _RUNS.clear()                            # one workload resident at a time
        _RUNS[name] = (wl, dev, got, out, L)
    return _RUNS[name]


GROUPS = {"C1": 1, "C2": 2, "C3": 4, "C4": 4, "V4": 2}


@pytest.mark.parametrize("name,part", [(n, p) for n, g in GROUPS.items() for p in range(g)])
def test_decode_config_every_row(name, part):
    wl, dev, got, out, L = _decode_run(name)
    nparts = GROUPS[name]
    reqs = list(range(part, wl.num_req, nparts))
    print(f"{name} part {part}/{nparts}: oracle on {len(reqs)} requests", flush=True)
    ref = oracle.pipeline.decode_logits(wl, requests=reqs)
    live = {r: v for r, v in ref.items() if len(v)}
    check_logits(got, live, label=name)
    sel = sorted(ref)
    check_topk_e2e(out[sel], {i: ref[r] for i, r in enumerate(sel)}, L[sel], wl.topk, label=name)
    # idx_topk on the oracle's fp32 logits (these rows; the others keep the
    # GPU's logits), with the batch's row descriptor: bit-exact
    buf = got.copy()
    for r, v in ref.items():
        buf[r, : len(v)] = v.astype(np.float32)
    rows = dev.decode_rows()
    o2 = torch.full((len(L), wl.topk), -7, dtype=torch.int32, device=dev.device)
    idx.idx_topk(torch.from_numpy(buf).to(dev.device), rows, wl.topk, o2, topk_workspace(rows, wl.topk))
    o2 = o2.cpu().numpy()
    for r in sel:
        exp = oracle.topk.topk_row(buf[r, : L[r]].astype(np.float64), int(L[r]), wl.topk)
        assert np.array_equal(o2[r], exp), f"{name} row {r} (L={L[r]}): top-k on oracle logits differs"


def _c5_sample(M):
    return sorted(set(range(0, M, 64)) | {M - 1})


@pytest.mark.parametrize("half", [0, 1])
def test_prefill_c5_chunks_sampled(half):
    if "C5" not in _RUNS:
        _RUNS.clear()
        wl = config("C5")
        _RUNS["C5"] = (wl, Dev(wl))
    wl, dev = _RUNS["C5"]
    recs = idx.idx_prefill_chunks(wl.seq_lens, wl.query_lens, 65536, 512 << 20)
    assert len(recs) == 16
    for ci in range(8 * half, 8 * half + 8):
        rec = recs[ci]
        rows = dev.prefill_rows(rec)
        M, N = rec["q_end"] - rec["q_begin"], rec["total_seq_lens"]
        q, w = dev.chunk_queries(rec)
        logits = torch.empty((M, N), device=dev.device)
        ws = topk_workspace(rows, wl.topk)
        print(f"C5 chunk {ci}: {M} rows x {N} columns", flush=True)
        idx.idx_logits_paged(dev.cache, rows, q, w, logits, ws)
        out = torch.full((M, wl.topk), -7, dtype=torch.int32, device=dev.device)
        idx.idx_topk(logits, rows, wl.topk, out, ws)
        torch.cuda.synchronize()
        assert idx.idx_read_device_status(ws) == 0
        req, j, L, ks, _ = oracle.pipeline.prefill_chunk_row_info(wl, rec)
        outc = out.cpu().numpy()
        check_topk_invariants(outc, L, wl.topk, label=f"C5 chunk {ci}")
        sample = _c5_sample(M)
        ref = oracle.pipeline.prefill_chunk_logits(wl, rec, sample_rows=sample)
        got = logits[sample].cpu().numpy()
        check_logits(got, {i: ref[r] for i, r in enumerate(sample)}, col0=ks[sample], check_untouched=False,
                     label=f"C5 chunk {ci}")
        check_topk_e2e(outc[sample], {i: ref[r] for i, r in enumerate(sample)}, L[sample], wl.topk,
                       label=f"C5 chunk {ci}")
        # idx_topk on the chunk's logits with the sampled rows replaced by the
        # oracle's fp32 values: those rows bit-exact
        for r in sample:
            c0 = int(ks[r])
            logits[r, c0 : c0 + len(ref[r])] = torch.from_numpy(ref[r].astype(np.float32)).to(dev.device)
        out2 = torch.full((M, wl.topk), -7, dtype=torch.int32, device=dev.device)
        idx.idx_topk(logits, rows, wl.topk, out2, ws)
        o2 = out2[sample].cpu().numpy()
        for i, r in enumerate(sample):
            exp = oracle.topk.topk_row(ref[r].astype(np.float32).astype(np.float64), int(L[r]), wl.topk)
            assert np.array_equal(o2[i], exp), f"C5 chunk {ci} row {r}: top-k on oracle logits differs"
        print(f"C5 chunk {ci} ok ({len(sample)} rows checked)", flush=True)
        del logits, out, out2
