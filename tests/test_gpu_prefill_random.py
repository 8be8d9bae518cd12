"""GPU: seeded random prefill batches through the planner, idx_logits_paged
on each chunk's PREFILL rows and idx_topk on the chunk's logits, against
the oracle.

Each case draws 1..8 requests (query lengths 0..seq_len, some requests
without queries), the key format (fp8 e4m3 at head_dim 32/64/128, MXFP4 at
128), 1..64 heads, k in 1..2048, a key-workspace size of at least the
longest request and a logits budget that often forces sub-chunks on the
query rows.  The planner's records must equal the oracle planner's; each
chunk's logits must match the oracle within 1e-4 + 2e-3 |oracle| at the
request's workspace offset (nothing written elsewhere) and its top-k rows
must be the oracle's up to keys within that tolerance of the k-th largest
logit.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_util import Dev, check_logits, check_topk_e2e
from tests.test_gpu_prefill import _chunks, _run_chunk
from workloads import build_prefill

pytestmark = pytest.mark.gpu


def _case(i):
    rng = np.random.default_rng(9300 + i)
    fmt = "mxfp4" if rng.random() < 0.3 else "fp8"
    D = int(rng.choice([32, 64, 128])) if fmt == "fp8" else 128
    H = int(rng.integers(1, 65))
    k = int(rng.choice([1, 3, 64, 257, 2048]))
    B = int(rng.integers(1, 9))
    seq = []
    for _ in range(B):
        kind = int(rng.integers(0, 4))
        if kind == 0:
            seq.append(64 * int(rng.integers(1, 30)) + int(rng.integers(-1, 2)))
        elif kind == 1:
            seq.append(int(rng.integers(0, 200)))
        else:
            seq.append(int(rng.integers(200, 6000)))
    seq = np.array(seq, dtype=np.int32)
    ql = np.array([int(rng.integers(0, min(int(s), 300) + 1)) if rng.random() < 0.85 else 0 for s in seq],
                  dtype=np.int32)
    if ql.sum() == 0:
        ql[int(np.argmax(seq))] = min(int(seq.max()), 17)
    ws_tokens = int(seq.max()) + int(rng.integers(0, 4000))
    budget = int(rng.choice([1 << 16, 1 << 18, 1 << 20, 1 << 24]))
    name = f"prand{i}-{fmt}-D{D}-H{H}-k{k}-B{B}"
    wl = build_prefill(seed=9300 + i, seq_lens=seq, query_lens=ql, heads=H, head_dim=D, topk=k, fmt=fmt,
                       w_std=1.0 / 8, name=name)
    return wl, ws_tokens, budget


@pytest.mark.parametrize("i", range(12))
def test_random_prefill_batch(i):
    wl, ws_tokens, budget = _case(i)
    recs = _chunks(wl, ws_tokens, budget)
    print(f"case {wl.name}: seq_lens {wl.seq_lens.tolist()} query_lens {wl.query_lens.tolist()} "
          f"workspace {ws_tokens} budget {budget}: {len(recs)} chunks", flush=True)
    dev = Dev(wl)
    for ci, rec in enumerate(recs):
        got, out, _ = _run_chunk(dev, rec)
        req, j, L, ks, _ = oracle.pipeline.prefill_chunk_row_info(wl, rec)
        ref = oracle.pipeline.prefill_chunk_logits(wl, rec)
        check_logits(got, ref, col0=ks, label=f"{wl.name} chunk {ci}")
        check_topk_e2e(out, ref, L, wl.topk, label=f"{wl.name} chunk {ci}")
