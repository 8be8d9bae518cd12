"""GPU: top-k of rows longer than 131072 keys, bit-exact against the oracle.

The pages size the indexer for max_model_len 163840 (the DeepSeek-V3.2
indexer page, get_max_prefill_buffer_size), so decode rows longer than the
selector's 131072-position bitmap are real.  Such rows take the streaming
selection's global refinement and ordered compaction from the row itself.
Both kernels that run it are covered: one 1024-thread workgroup per row
(batches of fewer than 512 rows) and the 512-thread kernel that batches of
at least two rows per CU run on every row.  Value patterns: random, heavy
ties with signed zeros, one value everywhere, a top value held by 40 % of the
keys, zeros with a few positives, infinities and huge magnitudes, ramps.
Every output row carries a slack row after it that must stay untouched.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from tests.gpu_util import topk_workspace

pytestmark = pytest.mark.gpu

LONG = [131073, 163840, 262144, 200003, 131073, 262144, 150001, 262144, 163840]


def _pattern(kind, L, rng):
    if L == 0:
        return np.zeros(0, dtype=np.float32)
    if kind == 0:
        return (rng.standard_normal(L) * 8).astype(np.float32)
    if kind == 1:
        v = (rng.integers(0, 8, size=L) * 0.5).astype(np.float32)
        v[rng.random(L) < 0.3] = -0.0
        return v
    if kind == 2:
        return np.full(L, 3.25, dtype=np.float32)
    if kind == 3:
        v = (rng.standard_normal(L) * 2).astype(np.float32)
        v = np.minimum(v, 6.0)
        v[rng.random(L) < 0.4] = 7.0          # the top value held by 40 % of the keys
        return v
    if kind == 4:
        v = np.where(rng.random(L) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        v[rng.integers(0, L, size=100)] = rng.random(100).astype(np.float32) + 1.0
        return v
    if kind == 5:
        v = np.clip(rng.standard_normal(L) * 1e38, -3.3e38, 3.3e38).astype(np.float32)
        v[::97] = np.inf
        v[5::89] = -np.inf
        return v
    if kind == 6:
        return np.arange(L, dtype=np.float32)            # the last k positions win
    if kind == 7:
        return (L - np.arange(L)).astype(np.float32)     # the first k positions win
    return (rng.integers(-3, 4, size=L) * 0.125).astype(np.float32)


def _run_rows(lens, vals, k):
    R = len(lens)
    stride = max(lens) + 5          # rows at unaligned addresses too
    buf = np.full((R, stride), np.nan, dtype=np.float32)
    for r, v in enumerate(vals):
        buf[r, : len(v)] = v
    d = torch.device("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device=d)
    bt = torch.zeros((R, 1), dtype=torch.int32, device=d)
    rows = idx.Rows.decode(bt, seq, max(lens))
    assert rows.num_rows == R
    logits = torch.from_numpy(buf).to(d)
    out = torch.full((R + 1, k), -7, dtype=torch.int32, device=d)       # one slack row
    ws = topk_workspace(rows, k, d)
    print(f"idx_topk: {R} rows, max L {max(lens)}, k {k}", flush=True)
    idx.idx_topk(logits, rows, k, out[:R], ws)
    got = out.cpu().numpy()
    assert (got[R] == -7).all(), "the selector wrote past the last output row"
    return got[:R]


@pytest.mark.parametrize("k", [1, 2048, 4096])
def test_rows_past_bitmap_small_batch(k):
    rng = np.random.default_rng(1000 + k)
    lens = list(LONG)
    vals = [_pattern(i % 9, L, rng) for i, L in enumerate(lens)]
    got = _run_rows(lens, vals, k)
    for r, v in enumerate(vals):
        exp = oracle.topk.topk_row(v.astype(np.float64), lens[r], k)
        assert np.array_equal(got[r], exp), f"row {r} (L={lens[r]}, pattern {r % 9}) differs"


@pytest.mark.parametrize("k", [1, 2048, 4096])
def test_rows_past_bitmap_lean_batch(k):
    """512 rows (two per CU): the streaming-only 512-thread kernel runs every
    row, long and short."""
    rng = np.random.default_rng(2000 + k)
    R = 512
    lens, vals = [], []
    short = [0, 1, k - 1, k, k + 1, 100, 3000, 20000, 32769, 70000]
    for r in range(R):
        if r % 16 == 0:
            L = LONG[(r // 16) % len(LONG)]
        else:
            L = max(0, short[r % len(short)])
        lens.append(L)
        vals.append(_pattern(r % 9, L, rng))
    got = _run_rows(lens, vals, k)
    for r, v in enumerate(vals):
        exp = oracle.topk.topk_row(v.astype(np.float64), lens[r], k)
        assert np.array_equal(got[r], exp), f"row {r} (L={lens[r]}, pattern {r % 9}) differs"


@pytest.mark.parametrize("k", [1, 64, 2048])
def test_sampled_selection_skewed_samples(k):
    """Rows whose systematic block sample (every 16th 64-key block for these
    lengths) misjudges the threshold: large values exactly on the sampled
    blocks (too few keys reach the sample's threshold) or small values there
    (too many): the one-read selection falls back, the rows stay exact;
    plus ordinary rows that take the one-read path.  512 rows: the
    streaming-only kernel."""
    rng = np.random.default_rng(3000 + k)
    R = 512
    lens, vals = [], []
    for r in range(R):
        L = [65536, 40000, 16384, 20000][r % 4]
        v = rng.standard_normal(L).astype(np.float32)
        blocks = np.arange(L) // 64
        on = blocks % 16 == 0
        kind = r % 3
        if kind == 0:
            v[on] = 100.0 + rng.random(on.sum()).astype(np.float32)
        elif kind == 1:
            v[on] = -100.0 - rng.random(on.sum()).astype(np.float32)
        lens.append(L)
        vals.append(v)
    got = _run_rows(lens, vals, k)
    for r, v in enumerate(vals):
        exp = oracle.topk.topk_row(v.astype(np.float64), lens[r], k)
        assert np.array_equal(got[r], exp), f"row {r} (L={lens[r]}, kind {r % 3}) differs"
